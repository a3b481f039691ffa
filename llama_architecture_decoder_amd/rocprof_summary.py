"""Summaries of rocprofv3 output for the batch-1 decode benchmark (kernel trace statistics and HBM traffic).

Usage (from the repository root, after the rocprofv3 runs given in profiles/decode_8b_hbm_traffic.md):

    python -m llama_architecture_decoder_amd.rocprof_summary traffic <fetch_dir> <write_dir> [out.json] [workload]

reads every ``*counter_collection.csv`` under the two directories (one FETCH_SIZE run, one WRITE_SIZE run of
``bench.py --copy-probe``), averages each counter per kernel over its dispatches, scales the counts by what
they read for the 1 GiB plain copy (``__amd_rocclr_copyBuffer``: 1 GiB fetched, 1 GiB written) and writes
the per-launch traffic of the decode kernels with the hash of the sources it was measured on (bench.py
reports ``traffic`` only while that hash still matches).  workload: decode_8b (default), decode_1_7b
(``bench.py --secondary-only``) or batched_8b (``bench.py --batched-only``, its attention).

    python -m llama_architecture_decoder_amd.rocprof_summary stats <kernel_stats.csv>

prints the kernel table (calls, average and total duration, share) of a ``--kernel-trace --stats`` run as
markdown.

    python -m llama_architecture_decoder_amd.rocprof_summary mfma <counter_dir>

prints, per matrix-core kernel of a ``--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 ...`` run,
the mean dispatch duration, the executed bf16 matrix FLOPs (MOPS x 512) per second and the busy fraction of
the matrix pipes (busy cycles summed over the 1024 SIMDs / (duration x 2.4 GHz x 1024)).
"""
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["llama_architecture_decoder_amd/csrc/gemv.hip", "llama_architecture_decoder_amd/csrc/gemv_body.h",
           "llama_architecture_decoder_amd/csrc/common.h"]
COPY = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30

# decode kernels per workload (substrings of the kernel names; bf16 weights: unsigned short)
KERNELS = {
    "decode_8b": {
        "gate_up": "k_gemv<unsigned short, 2, 2, true>",
        "down": "k_gemv<unsigned short, 7, 1, false>",
        "qkv_attention": "k_qkv_attn<unsigned short, 2, unsigned short, 128, 4>",
        "o_proj": "k_gemv<unsigned short, 2, 1, false>",
        "lm_head": "k_gemv<unsigned short, 2, 3, true>",
    },
    "decode_1_7b": {
        "gate_up": "k_gemv<float, 2, 2, true>",
        "down": "k_gemv<float, 8, 1, false>",
        "qkv_attention": "k_qkv_attn<float, 2, float, 64, 1>",
        "o_proj": "k_gemv<float, 2, 1, false>",
        "lm_head": "k_gemv<float, 2, 3, true>",
    },
    "batched_8b": {
        "attention": "k_attn_stream<128, 4>",
    },
}


def sources_hash() -> str:
    h = hashlib.sha256()
    for p in SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def counter_means(directory: str, counter: str, largest: str = ""):
    """{kernel name: (dispatches, mean counter value)} over every counter CSV under `directory`; for the
    kernel named `largest`, only its dispatches within 10% of its largest value (the 1 GiB copies, not the
    small uploads the same copy kernel also serves)."""
    per = defaultdict(dict)  # name -> dispatch id -> summed value (a counter may come in several rows)
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                d = (fn, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                per[name][d] = per[name].get(d, 0.0) + float(row["Counter_Value"])
    out = {}
    for k, v in per.items():
        vals = list(v.values())
        if largest and largest in k:
            vals = [x for x in vals if x >= 0.9 * max(vals)]
        out[k] = (len(vals), sum(vals) / len(vals))
    return out


def find(means, sub):
    hits = [(k, v) for k, v in means.items() if sub in k]
    if len(hits) != 1:
        raise KeyError(f"{len(hits)} kernels match {sub!r}")
    return hits[0][1]


def traffic(fetch_dir: str, write_dir: str, out: str, workload: str = "decode_8b"):
    sys.path.insert(0, ROOT)
    import bench
    import synth
    from synth import configs
    fm = counter_means(fetch_dir, "FETCH_SIZE", COPY)
    wm = counter_means(write_dir, "WRITE_SIZE", COPY)
    ff = COPY_BYTES / 1024 / find(fm, COPY)[1]
    wf = COPY_BYTES / 1024 / find(wm, COPY)[1]
    if workload == "decode_8b":
        cfg = configs.LLAMA31_8B
        t_mean = cfg.kv_fill + 4  # the mean position of the 8 profiled steps after one warm-up step
        alg = lambda cls: bench.kernel_bytes(cfg, cls, t_mean)
    elif workload == "decode_1_7b":
        # `bench.py --secondary-only --secondary-steps 16 --warmup 1`: the prompt's positions go through the
        # decode kernels too (F32 models prefill one position after another), then one warm-up step and
        # the timed and the profiled pass of 16 steps: the mean algorithmic bytes over those dispatches
        cfg = configs.SMOLLM2_1_7B
        P = cfg.prompt_len
        ts = list(range(P)) + [P] + 2 * list(range(P, P + 16))
        alg = lambda cls: int(round(sum(bench.kernel_bytes(cfg, cls, t) for t in ts) / len(ts)))
    else:  # batched_8b: every row's K/V rows 0..t per layer launch, at the mean step (warm-up 1 + 4 steps)
        cfg = configs.LLAMA31_8B_LONG
        lens = synth.row_lengths(cfg).astype("int64") + 3
        alg = lambda cls: int(sum(2 * cfg.kvw * cfg.kvbytes * (int(t) + 1) for t in lens))
    rec = {"workload": workload, "kernel": "gate_up", "sources": SOURCES, "sources_sha256_16": sources_hash(),
           "fetch_factor": ff, "write_factor": wf, "per_launch": {}}
    rows = []
    for cls, sub in KERNELS[workload].items():
        n, fk = find(fm, sub)
        _, wk = find(wm, sub)
        tb = (fk * ff + wk * wf) * 1024
        ab = alg(cls)
        rec["per_launch"][cls] = {"fetch_kib": fk, "write_kib": wk, "traffic_bytes": tb, "algorithmic_bytes": ab,
                                  "dispatches": n}
        rows.append(f"| {cls} (`{sub}`) | {n} | {fk:.1f} | {wk:.1f} | {tb:,.0f} | {ab:,} | {tb / ab:.3f} |")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"copy: FETCH_SIZE {find(fm, COPY)[1]:.1f} KiB, WRITE_SIZE {find(wm, COPY)[1]:.1f} KiB per 1 GiB dispatch "
          f"({find(fm, COPY)[0]} dispatches): fetch factor {ff:.4f}, write factor {wf:.4f}")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic (scaled) bytes | algorithmic bytes | "
          "traffic / algorithmic |")
    print("|---|---|---|---|---|---|---|")
    print("\n".join(rows))


def stats(fn: str):
    with open(fn, newline="") as f:
        rows = list(csv.DictReader(f))
    print("| kernel | calls | average us | total ms | % of GPU time |")
    print("|---|---|---|---|---|")
    for r in rows:
        name = r["Name"]
        name = name if len(name) <= 90 else name[:87] + "..."
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
              f"{float(r['Percentage']):.2f} |")


def mfma(directory: str, clock_ghz: float = 2.4, simds: int = 1024):
    per = defaultdict(lambda: defaultdict(dict))
    dur = {}
    for fn in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                k, d = row["Kernel_Name"], (fn, row["Dispatch_Id"])
                per[k][d][row["Counter_Name"]] = per[k][d].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
                dur[(k, d)] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    print("| kernel | dispatches | average us | executed bf16 matrix TFLOP/s | matrix pipes busy |")
    print("|---|---|---|---|---|")
    for k, ds in sorted(per.items(), key=lambda kv: -sum(dur[(kv[0], d)] for d in kv[1])):
        busy = sum(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for v in ds.values()) / len(ds)
        if busy <= 0:
            continue
        mops = sum(v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for v in ds.values()) / len(ds)
        t = sum(dur[(k, d)] for d in ds) / len(ds)
        name = k if len(k) <= 60 else k[:57] + "..."
        print(f"| `{name}` | {len(ds)} | {t / 1e3:.1f} | {mops * 512 / t / 1e3:.0f} | "
              f"{busy / (t * clock_ghz * simds):.3f} |")


if __name__ == "__main__":
    if len(sys.argv) >= 4 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3],
                sys.argv[4] if len(sys.argv) > 4 else os.path.join(ROOT, "profiles", "decode_8b_hbm_traffic.json"),
                sys.argv[5] if len(sys.argv) > 5 else "decode_8b")
    elif len(sys.argv) == 3 and sys.argv[1] == "stats":
        stats(sys.argv[2])
    elif len(sys.argv) == 3 and sys.argv[1] == "mfma":
        mfma(sys.argv[2])
    else:
        print(__doc__)
        sys.exit(2)
