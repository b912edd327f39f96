"""Turn rocprofv3 CSV output of a bench.py run into short text summaries.

Usage (on the machine that ran the profiles):

    python -m compressed_attention_turboquant_amd.profsummary \
        --workload C3 --trace DIR_T --fetch DIR_F --write DIR_W \
        --trace-cmd "..." --fetch-cmd "..." --write-cmd "..." --out profiles

DIR_T holds `<prefix>_kernel_stats.csv` from `rocprofv3 --kernel-trace --stats
--output-format csv`; DIR_F / DIR_W hold `<prefix>_counter_collection.csv`
from `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --copy-calibration`.  The 1 GiB device copy that bench.py runs after
its timed region (the runtime's copy-buffer kernel, dispatched after the last
library kernel) calibrates both counters: its known byte count divided by what
the counter reports gives the factor that turns a counter reading into bytes.

Writes `kernels_<workload>.md` (per-kernel durations), `traffic_<workload>.md`
(per-dispatch HBM bytes next to the algorithmic bytes), with --sq
`counters_<workload>.md` (instruction mix per wave, matrix-core and vector-ALU
busy, LDS bank conflicts from SQ counter runs) and, for bench.py,
`traffic_decode_<workload>.json` and `traffic_quantize_<workload>.json`, each
stamped with the digest of the kernel sources they were measured on.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30

# (tag, substring of the kernel name) for the launches one library call makes
DECODE_KERNELS = ("prerotate_ref", "decode_mfma_kernel", "decode_wide_kernel", "decode_split_ref", "decode_combine_ref",
                  "combine_kernel", "combine_rows128_kernel")
QUANT_KERNELS = ("quantize_mfma_kernel", "quantize_keys_qjl_kernel", "quantize_tile_ref", "quantize_fwht")
DEQUANT_KERNELS = ("dequant_mfma_kernel", "dequant_fwht_kernel", "dequant_qjl_kernel")


def strip_comments(src):
    """C/C++ source text without its comments and with runs of whitespace
    collapsed (string and character literals are kept as they are)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_sources_digest(csrc=None):
    """sha256 over the library's kernel and host sources (file names and code,
    comments left out), so that a profile stays matched to the code it was
    measured on across edits that change only comments."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(PKG, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                h.update(name.encode())
                h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def _one(directory, suffix):
    hits = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {directory}")
    return hits[0]


def _unmangle(name):
    """name<args> for a mangled library kernel whose template arguments are
    integers, float or _Float16 (the profiler leaves names with _Float16
    arguments mangled); the name unchanged if it is not of that form."""
    m = re.match(r"_ZN2tq12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name
    i = m.end()
    base = name[i:i + int(m.group(1))]
    i += int(m.group(1))
    if not name.startswith("I", i):
        return base
    i += 1
    args = []
    while i < len(name) and name[i] != "E":
        if name.startswith("Li", i):
            j = name.index("E", i)
            args.append(name[i + 2:j])
            i = j + 1
        elif name.startswith("DF16_", i):
            args.append("_Float16")
            i += 5
        elif name[i] in "fi":
            args.append({"f": "float", "i": "int"}[name[i]])
            i += 1
        else:
            return name
    return f"{base}<{', '.join(args)}>"


def _short(name):
    name = _unmangle(name).replace("tq::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0] if "(" in name and "<" not in name.split("(")[0][-2:] else name[:80]


def _is_lib(name):
    """True for the library's kernels, demangled (tq::...) or not (_ZN2tq...)."""
    return "tq::" in name or "_ZN2tq" in name


def kernel_stats(directory):
    rows = list(csv.DictReader(open(_one(directory, "kernel_stats.csv"))))
    return [r for r in rows if _is_lib(r["Name"])]


def counters(directory, counter):
    """Per-kernel list of counter values (KiB per dispatch) in dispatch order,
    plus the copy-buffer dispatches that follow the last library dispatch."""
    rows = [r for r in csv.DictReader(open(_one(directory, "counter_collection.csv")))
            if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    last_tq = max(int(r["Dispatch_Id"]) for r in rows if _is_lib(r["Kernel_Name"]))
    per = collections.defaultdict(list)
    copy = 0.0
    for r in rows:
        v = float(r["Counter_Value"])
        if _is_lib(r["Kernel_Name"]):
            per[r["Kernel_Name"]].append(v)
        elif int(r["Dispatch_Id"]) > last_tq and "copyBuffer" in r["Kernel_Name"]:
            copy += v
    if copy <= 0:
        raise SystemExit(f"{counter}: no calibration copy after the library kernels")
    return per, COPY_BYTES / (copy * 1024.0)


def sq_counters(directories):
    """Per-kernel mean of every counter in the given --pmc runs' CSVs (library
    kernels only): {kernel name: {counter: mean per dispatch}}."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in directories:
        for r in csv.DictReader(open(_one(d, "counter_collection.csv"))):
            if _is_lib(r["Kernel_Name"]):
                per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in per.items()}


# (counter, what it says) for the summary table; per-wave figures divide by SQ_WAVES.
SQ_PER_WAVE = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD")


def counters_table(cfg, sq, digest, cmds):
    lines = [f"# Shader counters per dispatch, workload {cfg.name}", "",
             f"Kernel sources digest: `{digest}`", "",
             "Commands (from the repository root, TMPDIR=/tmp), one counter set per run:", "", "```"]
    lines += list(cmds) + ["```", "",
                           "Summary written by `python -m compressed_attention_turboquant_amd.profsummary`.", "",
                           "Per wave: instructions issued by one wave (SQ_INSTS_* / SQ_WAVES).  MfmaUtil: "
                           "matrix-core busy cycles over GPU-busy cycles x SIMDs (%).  VALUBusy: vector-ALU "
                           "busy (%).  LDS conflict: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE, the share "
                           "of LDS-active cycles lost to bank conflicts.", "",
                           "| kernel | waves | VALU / wave | MFMA / wave | LDS / wave | SALU / wave | "
                           "VMEM rd / wave | MfmaUtil % | VALUBusy % | LDS conflict |",
                           "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for name in sorted(sq):
        c = sq[name]
        w = c.get("SQ_WAVES", 0.0)
        per_wave = [f"{c[k] / w:.0f}" if w and k in c else "-" for k in SQ_PER_WAVE]
        util = f"{c['MfmaUtil']:.1f}" if "MfmaUtil" in c else "-"
        busy = f"{c['VALUBusy']:.1f}" if "VALUBusy" in c else "-"
        conf = (f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.3f}"
                if c.get("SQ_LDS_IDX_ACTIVE") else "-")
        lines.append(f"| `{_short(name)}` | {w:.0f} | " + " | ".join(per_wave) + f" | {util} | {busy} | {conf} |")
    return lines


def packed_bytes(cfg):
    k = cfg.d * cfg.k_bits // 8 + 4 + (cfg.d // 8 + 4 if cfg.k_qjl else 0)
    v = cfg.d * cfg.v_bits // 8 + 4
    return k, v


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--trace-cmd", required=True)
    ap.add_argument("--fetch-cmd", required=True)
    ap.add_argument("--write-cmd", required=True)
    ap.add_argument("--sq", nargs="*", default=[], help="directories of --pmc runs with SQ counters")
    ap.add_argument("--sq-cmd", nargs="*", default=[], help="the commands of those runs")
    ap.add_argument("--out", default="profiles")
    a = ap.parse_args()

    import sys
    sys.path.insert(0, os.path.dirname(PKG))
    import workloads
    cfg = workloads.CONFIGS[a.workload]
    digest = kernel_sources_digest()
    os.makedirs(a.out, exist_ok=True)

    stats = kernel_stats(a.trace)
    lines = [f"# Kernel durations, workload {cfg.name}", "",
             f"{workloads.WORKLOAD_TEXT[cfg.name]}", "",
             f"Kernel sources digest: `{digest}`", "", "Command (from the repository root, TMPDIR=/tmp):", "", "```",
             a.trace_cmd, "```", "", "Summary written by `python -m compressed_attention_turboquant_amd.profsummary`.", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    dec_sum = 0.0
    for r in stats:
        avg = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {avg:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {r['Percentage']}% |")
        if any(k in r["Name"] for k in DECODE_KERNELS):
            dec_sum += avg
    kb, vb = packed_bytes(cfg)
    rows = cfg.B * cfg.Hkv * cfg.N
    lines += ["", f"Sum of the decode call's kernel averages: {dec_sum:.1f} us; packed KV read "
              f"{(kb + vb) * rows / 1e9:.4f} GB, i.e. {(kb + vb) * rows / dec_sum / 1e3:.0f} GB/s "
              "over the kernels alone."]
    with open(os.path.join(a.out, f"kernels_{cfg.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    fetch, ff = counters(a.fetch, "FETCH_SIZE")
    write, fw = counters(a.write, "WRITE_SIZE")
    in_b = 2 if cfg.dtype == "f16" else 4
    algo = {"decode": (kb + vb) * rows,
            "quantize K": rows * (cfg.d * in_b + kb), "quantize V": rows * (cfg.d * in_b + vb),
            # codes and norm in, rows of the input's dtype out (QJL signs are not read)
            "dequantize": rows * (cfg.d * (cfg.k_bits + cfg.v_bits) // 8 + 8 + 2 * cfg.d * in_b)}
    t = [f"# HBM traffic per dispatch, workload {cfg.name}", "",
         f"Kernel sources digest: `{digest}`", "", "Commands (from the repository root, TMPDIR=/tmp):", "",
         "```", a.fetch_cmd, a.write_cmd, "```", "",
         "Summary written by `python -m compressed_attention_turboquant_amd.profsummary`.", "",
         f"Calibration with the 1 GiB device copy bench.py runs after its timed region: "
         f"FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f} give bytes.", "",
         "| kernel | dispatches | read (MB) | written (MB) |", "|---|---:|---:|---:|"]
    per_kernel = {}
    for name in sorted(set(fetch) | set(write)):
        fr = fetch.get(name, [0.0])
        wr = write.get(name, [0.0])
        rb = sum(fr) / len(fr) * 1024 * ff
        wb = sum(wr) / len(wr) * 1024 * fw
        per_kernel[name] = (rb, wb)
        t.append(f"| `{_short(name)}` | {len(fr)} | {rb / 1e6:.2f} | {wb / 1e6:.2f} |")

    def total(keys, which=None):
        tot = 0.0
        for name, (rb, wb) in per_kernel.items():
            if any(k in name for k in keys) and (which is None or which(name)):
                tot += rb + wb
        return tot

    dec = total(DECODE_KERNELS)
    quant = total(QUANT_KERNELS)
    deq = total(DEQUANT_KERNELS)
    t += ["", f"Decode call (all its launches): {dec / 1e9:.4f} GB moved vs {algo['decode'] / 1e9:.4f} GB "
          "of packed KV (algorithmic).",
          f"Quantize K + V calls: {quant / 1e9:.4f} GB moved vs "
          f"{(algo['quantize K'] + algo['quantize V']) / 1e9:.4f} GB (input rows in, packed rows out).",
          f"Dequantize K + V calls: {deq / 1e9:.4f} GB moved vs {algo['dequantize'] / 1e9:.4f} GB "
          "(codes and norms in, rows out)."]
    with open(os.path.join(a.out, f"traffic_{cfg.name}.md"), "w") as f:
        f.write("\n".join(t) + "\n")
    for tag, val, alg in (("decode", dec, algo["decode"]),
                          ("quantize", quant, algo["quantize K"] + algo["quantize V"]),
                          ("dequantize", deq, algo["dequantize"])):
        with open(os.path.join(a.out, f"traffic_{tag}_{cfg.name}.json"), "w") as f:
            json.dump({"workload": cfg.name, "sources_digest": digest, "bytes_per_launch": round(val),
                       "algorithmic_bytes_per_launch": alg, "fetch_factor": round(ff, 4),
                       "write_factor": round(fw, 4), "commands": [a.fetch_cmd, a.write_cmd]}, f, indent=1)
    if a.sq:
        c = counters_table(cfg, sq_counters(a.sq), digest, a.sq_cmd)
        with open(os.path.join(a.out, f"counters_{cfg.name}.md"), "w") as f:
            f.write("\n".join(c) + "\n")
        t += [""] + c
    print("\n".join(lines + [""] + t))


if __name__ == "__main__":
    main()
