"""Benchmark: one decode round's verify + P-EAGLE batch build on one MI355X.

A step is one pass of the whole path over one batch: spec_verify_sample on
B=1024 sequences with K=7 drafts over a V=151936 bf16 vocabulary (logits
2.49 GB, draft probabilities 4.36 GB, both resident in HBM), then
peagle_build_draft_batch (H=2048 bf16) fed by the verify outputs on the same
stream.  The greedy variant of the same step is timed too and reported in
"greedy_step".

Prints one JSON line.  `value` is verified logit rows per second, B*(K+1)
rows per step.  `roofline` covers the dominant kernel (the sampled verify),
timed with HIP events on the stream it runs on; `cpu_baseline` times the
fp64 CPU oracle on the host over as much of the same batch as fits a time
budget.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
TRACE_EVERY = 4                # the timed loop traces the dominant kernel in every 4th step
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_verify_sample_fused_b1024.json")
CEILING_LIB = os.path.join(ROOT, "draft_verification_vocab_amd", "libsvceiling.so")


@contextlib.contextmanager
def quiet_host():
    """A timed region without Python garbage collection: a full collection
    over the objects torch and the input generators leave behind takes tens
    of milliseconds, long enough to stall the enqueue of a short timed loop."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of CPU oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--no-greedy", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the captured step graph")
    ap.add_argument("--no-round", action="store_true",
                    help="skip timing the decode round on the two q interfaces")
    ap.add_argument("--no-tree", action="store_true",
                    help="skip timing draft-tree verification")
    ap.add_argument("--no-small", action="store_true",
                    help="skip timing the mid-size verify, the P-EAGLE build, the "
                         "large-vocabulary verify workloads and the fp32-logit verify")
    ap.add_argument("--no-early-exit", action="store_true",
                    help="skip the early-exit verify comparison")
    ap.add_argument("--no-draft", action="store_true",
                    help="skip timing the drafter-output sampling kernel")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run only this many untimed steps (for rocprofv3) and exit; inputs are "
                         "then drawn in this process (no worker processes under a profiler)")
    ap.add_argument("--profile-workload", choices=("fused", "large-vocab"), default="fused",
                    help="with --profile-steps: the fused B=1024 step and the comparison kernels "
                         "(fused), or the B=64 K=7 V=201088 bf16 verify over four rotated "
                         "input copies (large-vocab)")
    ap.add_argument("--hash-out", default=None,
                    help="with --profile-steps: write the kernel source hash of this run here")
    ap.add_argument("--ingest-valu", default=None, metavar="VALU_CSV",
                    help="write profiles/valu_counters_fused_b1024.md from a --pmc SQ_INSTS_VALU "
                         "SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE run")
    ap.add_argument("--ingest-trace", nargs="+", metavar="FILE",
                    help="write the kernel trace summary under profiles/ from a rocprofv3 "
                         "kernel-trace CSV (and the log of a bench run on the same sources)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE runs of --profile-steps) into the traffic record and exit")
    ap.add_argument("--workers", type=int, default=None,
                    help="processes drawing the synthetic inputs (default: one per core, up to 16)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the HIP sources the timed kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_verification_vocab_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def verify_bytes(B, K, V, zsize, acc, sample=True):
    """Algorithmic HBM bytes of a verify call, split as (row kernel, the rest).

    Row kernel: every logit row once.  The rest (accept scan, and for sampling
    the draw): the draft tokens, the outputs, and for sampling the q(d) / z(d)
    gathers, the uniforms, p_k(d_k) and the drafter's row a_b of each sequence
    that rejects a draft.
    The draw's second read of logit row a is not counted: the method reads
    every logit once."""
    rows = B * (K + 1) * V * zsize
    scan = B * K * 4 + B * (K + 1) * 4 + B * 4          # draft tokens, out_tokens, num_accepted
    if sample:
        scan += B * K * 4 * 2                           # q(d) and z(d) gathers
        scan += B * (K + 1) * 4                         # uniforms
        scan += B * K * 4                               # p_k(d_k) output
        scan += int((acc < K).sum()) * V * 4            # q row a_b of rejecting sequences
    return rows, scan


def build_bytes(B, K, H, hsize):
    """Algorithmic HBM bytes of one build launch: every verify hidden row read
    once, h_shared, the 2K output rows per sequence and their metadata."""
    n = B * (K + 1) * H * hsize + H * hsize + B * 2 * K * H * hsize
    n += B * ((K + 1) * 4 + 4 + K * 4 + 8 + 8)      # verify outputs, draft tokens, L, table reads
    n += B * 2 * K * (4 + 8 + 8) + B * K * 4         # ids, positions, slots, sample rows
    return n


def cpu_baseline(vi, bi, budget_s):
    """The oracle as it stands, one thread, over the batch until the budget runs out."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    K = vi.spec.K
    with threadpool_limits(1):
        t0 = time.perf_counter()
        done = _oracle_loop(oracle, np, vi, bi, K, t0, budget_s)
        dt = time.perf_counter() - t0
    rows = done * (K + 1)
    return {"value": rows / dt, "unit": "verified logit rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {vi.spec.B} sequences of the same batch "
                      f"(sampled verify + P-EAGLE build per sequence, fp64 numpy), {dt:.1f} s"}


_SHARED = {}                   # the inputs, shared with forked oracle workers


def _oracle_worker(args):
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    seqs, K = args
    vi, bi = _SHARED["vi"], _SHARED["bi"]
    with threadpool_limits(1):
        for b in seqs:
            z = oracle.decode_logits(vi.logits[b], "bf16")
            tr = oracle.verify_sample_seq(z, vi.draft_probs[b], vi.draft_tokens[b],
                                          vi.uniforms[b], vi.temperature)
            oracle.build_draft_batch(tr.out_tokens[None], np.array([tr.a], np.int32),
                                     vi.draft_tokens[b:b + 1], bi.start_pos[b:b + 1],
                                     bi.block_table[b:b + 1], bi.spec.block_size,
                                     bi.target_hidden[b * (K + 1):(b + 1) * (K + 1)], bi.h_shared,
                                     bi.mask_token_id)
    return len(seqs)


def cpu_baseline_all_cores(vi, bi, workers):
    """The same oracle over the whole batch, sequences split across forked
    processes (one thread each).  Runs before anything touches the GPU: the
    workers share the inputs with this process copy-on-write."""
    import multiprocessing as mp
    n = max(1, workers)
    _SHARED["vi"], _SHARED["bi"] = vi, bi
    K = vi.spec.K
    chunks = [(list(range(i, vi.spec.B, n)), K) for i in range(n)]
    with mp.get_context("fork").Pool(n) as pool:
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_worker, chunks))
        dt = time.perf_counter() - t0
    _SHARED.clear()
    return {"value": done * (K + 1) / dt, "unit": "verified logit rows/s", "cores": n,
            "kind": "oracle",
            "sample": f"all {done} sequences of the same batch split across {n} processes "
                      f"(sampled verify + P-EAGLE build per sequence, fp64 numpy), {dt:.2f} s"}


def _oracle_loop(oracle, np, vi, bi, K, t0, budget_s):
    done = 0
    for b in range(vi.spec.B):
        z = oracle.decode_logits(vi.logits[b], "bf16")
        tr = oracle.verify_sample_seq(z, vi.draft_probs[b], vi.draft_tokens[b], vi.uniforms[b],
                                      vi.temperature)
        oracle.build_draft_batch(tr.out_tokens[None], np.array([tr.a], np.int32),
                                 vi.draft_tokens[b:b + 1], bi.start_pos[b:b + 1],
                                 bi.block_table[b:b + 1], bi.spec.block_size,
                                 bi.target_hidden[b * (K + 1):(b + 1) * (K + 1)], bi.h_shared,
                                 bi.mask_token_id)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    return done


COPY_BYTES = 1 << 30           # the calibration copy of --profile-steps


def _library_kernel(name):
    """A kernel of the verify library (namespace sv) or of the comparison
    library (an anonymous namespace at file scope), not one of torch's."""
    return (name.startswith(("void sv::", "sv::", "void (anonymous namespace)::",
                             "(anonymous namespace)::")) and "at::" not in name)


def _profile_record(csv_path):
    """(kernel source hash, workload) that a profiled run wrote with
    --hash-out into source_hash.txt next to its CSV."""
    hp = os.path.join(os.path.dirname(csv_path), "source_hash.txt")
    if not os.path.exists(hp):
        sys.exit(f"{hp} is missing: cannot tell which kernels {csv_path} measured")
    words = open(hp).read().split()
    return words[0], (words[1] if len(words) > 1 else "fused")


def ingest_counters(fetch_csv, write_csv):
    """Per-kernel HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the 1 GiB copy
    in the same run; writes the traffic record and a markdown summary.  Both
    profiled runs must have recorded (--hash-out source_hash.txt next to their
    CSV) the kernel source hash of the current sources."""
    here = kernel_source_hash()
    workloads = set()
    for csv in (fetch_csv, write_csv):
        got, wl = _profile_record(csv)
        if got != here:
            sys.exit(f"counters in {csv} were taken on kernel sources {got}, not the current {here}")
        workloads.add(wl)
    if len(workloads) != 1:
        sys.exit("the FETCH_SIZE and WRITE_SIZE runs profiled different workloads")
    workload = workloads.pop()
    import csv
    import collections

    def load(path, counter):
        # per (kernel, grid size): one kernel serves several workloads
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                per[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]) * 1024.0)
        return per

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k[0]]
    f_scale = COPY_BYTES / max(max(fetch[k]) for k in copy)
    w_scale = COPY_BYTES / max(max(write[k]) for k in copy)
    kernels = {}
    for key in sorted(fetch, key=lambda k: (k[0], -k[1])):
        name, grid = key
        if not _library_kernel(name):
            continue
        f = sum(fetch[key]) / len(fetch[key]) * f_scale
        w = sum(write.get(key, [0.0])) / max(1, len(write.get(key, []))) * w_scale
        kernels[f"{name} [grid {grid}]"] = {"fetch_bytes": f, "write_bytes": w,
                                            "hbm_bytes_per_launch": f + w,
                                            "dispatches": len(fetch[key]), "grid": grid}
    # the sampled row kernel of the workload: the largest grid of that kernel
    dom = max((k for k in kernels if "verify_rows<unsigned short, 1, true>" in k),
              key=lambda k: kernels[k]["grid"])
    rec = {"source_hash": kernel_source_hash(), "fetch_scale": f_scale, "write_scale": w_scale,
           "kernel": dom, "hbm_bytes_per_launch": kernels[dom]["hbm_bytes_per_launch"],
           "kernels": kernels}
    if workload == "fused":
        # the bench line's roofline.traffic comes from this record
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        md = os.path.join(ROOT, "profiles", "hbm_counters_fused_b1024.md")
        title = "fused step, B=1024 K=7 V=151936 bf16, H=2048"
        extra = ""
    else:
        md = os.path.join(ROOT, "profiles", "hbm_counters_large_vocab_b64.md")
        title = "large-vocabulary verify, B=64 K=7 V=201088 bf16, four rotated input copies"
        extra = " --profile-workload large-vocab"
    # the commands that made the two CSVs: one counter per profiler run, output
    # in the directory holding each CSV
    fdir, wdir = os.path.dirname(fetch_csv), os.path.dirname(write_csv)
    fo = os.path.basename(fetch_csv).split("_counter_collection")[0]
    wo = os.path.basename(write_csv).split("_counter_collection")[0]
    lines = [f"# HBM bytes per launch from rocprofv3 counters: {title}\n",
             "Commands (one counter per run, from /tmp with TMPDIR=/tmp; REPO = the repository root):\n",
             "```",
             f"timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/{fdir} -o {fo} -- python3 $REPO/bench.py --profile-steps 2{extra} --hash-out $REPO/{fdir}/source_hash.txt",
             f"timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/{wdir} -o {wo} -- python3 $REPO/bench.py --profile-steps 2{extra} --hash-out $REPO/{wdir}/source_hash.txt",
             f"python bench.py --ingest-counters {fetch_csv} {write_csv}",
             "```\n",
             f"Calibration (a plain 1 GiB device copy in the same runs): FETCH_SIZE x {f_scale:.4f}, "
             f"WRITE_SIZE x {w_scale:.4f} give bytes.  Kernel source hash `{rec['source_hash']}`.\n",
             "| kernel [grid size in threads] | dispatches | HBM read (GB) | HBM write (GB) | total (GB) |", "|---|---|---|---|---|"]
    for name, k in kernels.items():
        lines.append(f"| `{name}` | {k['dispatches']} | {k['fetch_bytes'] / 1e9:.4f} | "
                     f"{k['write_bytes'] / 1e9:.4f} | {k['hbm_bytes_per_launch'] / 1e9:.4f} |")
    if workload != "fused":
        lines.append("\nThe row kernel's algorithmic bytes are every logit row once: 64 x 8 x "
                     "201088 x 2 B = 0.2059 GB per launch.  FETCH_SIZE counts what leaves the "
                     "GPU's L2 for the memory fabric, so reads served by the 256 MB memory-side "
                     "Infinity Cache count as HBM reads here; the rotation over four input copies "
                     "(0.82 GB of logits) keeps the calls from finding their inputs cached.")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"traffic_file": TRAFFIC_FILE if workload == "fused" else None,
                      "summary": md, "dominant_hbm_bytes_per_launch": rec["hbm_bytes_per_launch"]}))


def ingest_trace(trace_csv, bench_log=None):
    """Kernel trace summary from rocprofv3's per-dispatch records: average,
    minimum and maximum duration per kernel and grid size (one kernel serves
    several workloads), the run's kernel source hash (--hash-out
    source_hash.txt next to the CSV), and, given the log of a `python
    bench.py` run on the same sources, its tracer's per-kernel times."""
    import csv
    import collections

    here = kernel_source_hash()
    got, _ = _profile_record(trace_csv)
    if got != here:
        sys.exit(f"the trace in {trace_csv} was taken on kernel sources {got}, not the current {here}")
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        name = r["Kernel_Name"]
        if not (_library_kernel(name) or "copyBuffer" in name):
            continue                 # torch's own kernels (input uploads, fills)
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        per[(name, grid)].append(us)
    rows = sorted(per.items(), key=lambda kv: -sum(kv[1]) / len(kv[1]))
    tdir = os.path.dirname(trace_csv)
    to = os.path.basename(trace_csv).split("_kernel_trace")[0]
    lines = ["# Kernel trace: fused high-concurrency step (B=1024, K=7, V=151936 bf16; build H=2048)\n",
             "Commands (from /tmp with TMPDIR=/tmp; REPO = the repository root):\n",
             "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/{tdir} -o {to} -- "
             f"python3 $REPO/bench.py --profile-steps 5 --hash-out $REPO/{tdir}/source_hash.txt",
             f"python bench.py --ingest-trace {trace_csv}" + (f" {bench_log}" if bench_log else ""),
             "```\n",
             "`--profile-steps 5` runs, five times on the B=1024 K=7 V=151936 bf16 inputs: a sampled, a greedy and "
             "a mixed verify each followed by the build, the drafter sampling with dense q and with "
             "row descriptors, the verify from drafter logits, the drafter sampling at per-sequence "
             "temperatures with row descriptors, the mixed verify from drafter logits, the "
             "early-exit sampled and greedy verify (`verify_rows_level`, four ranges each, the "
             "last three after a `verify_level_gate`) and "
             "the acceptance metrics; then the "
             "fused build and the two-kernel build of the comparison library (`meta_kernel`, "
             "`copy_kernel`) five times each on the same verify outputs and at the B=64 H=2880 build "
             "workload, the comparison library's drafter-bytes kernels (`rows_to_f32`, "
             "`write_rows`; 4 calls each), five greedy and five sampled tree verifications (64 "
             "trees of 15 nodes, V=151936 bf16), each also in its early-exit form "
             "(`tree_walk<…, true>` as the last template argument: no row kernel), five mixed "
             "tree verifications (per-tree temperatures, `tree_walk<…, 2, …>`), one drafter "
             "sampling of one row per tree node "
             "with row descriptors and five tree verifications from those drafter logits, "
             "one pass each of the read-ceiling kernel "
             "(`stream_read<true>` non-temporal, `stream_read<false>` cached) over the 2.49 GB "
             "logit buffer, and one 1 GiB copy (the counter calibration).\n",
             f"Kernel source hash (bench.py `kernel_source_hash`): `{here}`\n",
             "Per kernel and grid size (threads), from the per-dispatch records of the run "
             "(the `--stats` table averages one kernel over every grid it ran at):\n",
             "| kernel | grid | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|---|"]
    for (name, grid), v in rows:
        lines.append(f"| `{name}` | {grid} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | "
                     f"{max(v):.1f} |")
    # the sampled row kernel of the 8192-row batch: its largest grid
    dom = sorted(((grid, v) for (name, grid), v in per.items()
                  if "verify_rows<unsigned short, 1, true>" in name), key=lambda gv: -gv[0])
    if dom:
        grid, v = dom[0]
        lines.append(f"\nDominant kernel (`verify_rows<unsigned short, 1, true>`, the 8192-row fused "
                     f"batch, grid {grid}): {sum(v) / len(v):.1f} µs average over {len(v)} "
                     "dispatches (sampled verify and verify from drafter logits).")
    if bench_log:
        res = json.loads([ln for ln in open(bench_log) if ln.startswith("{")][-1])
        if res.get("kernel_source_hash") != here:
            sys.exit(f"{bench_log} was measured on other kernel sources")
        lines += ["\nSame sources, bench.py's tracer (HIP events on the kernels' stream, one "
                  f"kernel traced per loop, {res['steps']} timed steps of `python bench.py`):\n",
                  "| kernel | avg µs | algorithmic GB | GB/s | % of 8 TB/s |", "|---|---|---|---|---|"]
        for k, v in res["kernels"].items():
            lines.append(f"| {k} | {v['avg_ms'] * 1e3:.1f} | {v['algorithmic_bytes'] / 1e9:.4f} | "
                         f"{v['gbs']:.0f} | {v['frac'] * 100:.1f} |")
        g = res.get("greedy_step")
        if g:
            r = g["verify_greedy_rows"]
            lines.append(f"| verify_greedy_rows | {r['avg_ms'] * 1e3:.1f} | "
                         f"{r['algorithmic_bytes'] / 1e9:.4f} | {r['gbs']:.0f} | "
                         f"{r['frac'] * 100:.1f} |")
            lines.append(f"| verify_greedy_accept | {g['verify_greedy_accept_ms'] * 1e3:.1f} | | | |")
        lines.append(f"\nSampled step: {res['ms_per_step']:.3f} ms, {res['value'] / 1e6:.2f} M "
                     f"verified logit rows/s, {res['step_hbm_gbs']:.0f} GB/s algorithmic "
                     f"({res['step_hbm_frac'] * 100:.1f}% of 8 TB/s)" +
                     (f"; greedy step: {g['ms_per_step']:.3f} ms, {g['value'] / 1e6:.2f} M rows/s "
                      f"({g['step_hbm_frac'] * 100:.1f}%)." if g else "."))
        c = res.get("read_ceiling")
        if c:
            lines.append(f"\nRead ceiling (the plain streaming-read kernel over the same 2.489 GB "
                         f"logit buffer): non-temporal loads {c['nontemporal_gbs']:.0f} GB/s, cached "
                         f"loads {c['cached_gbs']:.0f} GB/s; the sampled row kernel reaches "
                         f"{res['roofline']['frac_of_read_ceiling'] * 100:.1f}% of the non-temporal "
                         "rate.")
    md = os.path.join(ROOT, "profiles", "kernel_trace_fused_b1024.md")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"summary": md, "kernels": len(rows)}))


def ingest_valu(valu_csv):
    """ALU load per kernel from instruction counters: VALU and fp32
    transcendental wave instructions per dispatch, converted to SIMD cycles
    (a wave64 instruction: 4 cycles on a 16-lane SIMD without packed fp32; a
    transcendental: 16, a quarter rate) and set against the SIMD cycles of the
    kernel's duration at 2.4 GHz (durations of the same dispatches, from the
    counter run's timestamps)."""
    import csv
    import collections
    if _profile_record(valu_csv)[0] != kernel_source_hash():
        sys.exit(f"{valu_csv}: counters not taken on the current kernel sources")
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    span = collections.defaultdict(dict)       # dispatch -> duration (us)
    for r in csv.DictReader(open(valu_csv)):
        key = (r["Kernel_Name"], int(r["Grid_Size"]))
        per[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        span[key][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    simd_cycles_per_us = 256 * 4 * 2400.0
    lines = ["# ALU load from instruction counters: fused-step kernels (B=1024, K=7, V=151936 bf16)\n",
             "Command (REPO = the repository root):\n", "```",
             f"timeout -s KILL 300 rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE --output-format csv -d $REPO/{os.path.dirname(valu_csv)} -o valu -- python3 $REPO/bench.py --profile-steps 2 --hash-out $REPO/{os.path.dirname(valu_csv)}/source_hash.txt",
             f"python bench.py --ingest-valu {valu_csv}", "```\n",
             "Counts are wave instructions per dispatch.  SIMD cycles: 4 per VALU instruction of a wave64 "
             "on a 16-lane SIMD (fp32 without packed math), 16 per transcendental (quarter rate).  "
             "Load = those cycles / (1024 SIMDs x duration x 2.4 GHz), durations from the "
             "counter run's own dispatch timestamps; exp/s counts lanes.\n",
             f"Kernel source hash `{kernel_source_hash()}`.\n",
             "| kernel [grid] | VALU instr | of which exp (fp32 transcendental) | duration µs | exp/s | ALU load at 2.4 GHz |",
             "|---|---|---|---|---|---|"]
    for (name, grid), c in sorted(per.items()):
        if not (name.startswith(("void sv::", "sv::")) or "stream_read<" in name) \
                or not c["SQ_INSTS_VALU"]:
            continue
        valu = sum(c["SQ_INSTS_VALU"]) / len(c["SQ_INSTS_VALU"])
        tr = sum(c["SQ_INSTS_VALU_TRANS_F32"]) / max(1, len(c["SQ_INSTS_VALU_TRANS_F32"]))
        us = sum(span[(name, grid)].values()) / len(span[(name, grid)])
        cycles = (valu - tr) * 4 + tr * 16
        lines.append(f"| `{name} [{grid}]` | {valu:.3e} | {tr:.3e} | {us:.1f} | "
                     f"{tr * 64 / (us * 1e-6):.2e} | {100 * cycles / (simd_cycles_per_us * us):.0f}% |")
    md = os.path.join(ROOT, "profiles", "valu_counters_fused_b1024.md")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(md)


def _stream_read_fn():
    import ctypes
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is not built (run __graft_entry__.build())")
    fn = ctypes.CDLL(CEILING_LIB).svc_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def _ceiling_fn(name, argtypes):
    import ctypes
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is not built (run __graft_entry__.build())")
    fn = getattr(ctypes.CDLL(CEILING_LIB), name)
    fn.argtypes = argtypes
    fn.restype = ctypes.c_int
    return fn


def draft_ceiling(torch, z_rows, rows, qbuf, reps):
    """The drafter's bytes without its arithmetic: plain kernels that read
    the gathered bf16 rows and write them back as fp32 (non-temporal and
    ordinary stores), and that only write the fp32 rows, over the same device
    buffers as the drafter sampling with q."""
    import ctypes
    vp, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    cvt = _ceiling_fn("svc_rows_to_f32", [vp, vp, i64, vp, i64, i, i, vp])
    wr = _ceiling_fn("svc_write_rows", [vp, i64, i, i, vp])
    n_out, V = rows.numel(), z_rows.shape[1]
    stream = torch.cuda.current_stream()
    calls = {
        "rows_to_f32_nontemporal": lambda: cvt(z_rows.data_ptr(), rows.data_ptr(), z_rows.shape[0],
                                               qbuf.data_ptr(), n_out, V, 1, stream.cuda_stream),
        "rows_to_f32_cached": lambda: cvt(z_rows.data_ptr(), rows.data_ptr(), z_rows.shape[0],
                                          qbuf.data_ptr(), n_out, V, 0, stream.cuda_stream),
        "write_rows_nontemporal": lambda: wr(qbuf.data_ptr(), n_out, V, 1, stream.cuda_stream),
        "write_rows_cached": lambda: wr(qbuf.data_ptr(), n_out, V, 0, stream.cuda_stream)}
    out = {"kernels": "rows_to_f32: one 512-thread workgroup per output row reads the gathered "
                      "bf16 row (16-byte non-temporal loads) and writes it as fp32; write_rows: "
                      "the fp32 rows written alone"}
    for key, fn in calls.items():
        for _ in range(3):
            if fn():
                raise RuntimeError(f"{key} failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = n_out * V * (6 if key.startswith("rows") else 4)
        out[key] = {"ms": ms, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9}
    return out


def split_build(torch, o, a, d, L, bt, block_size, hid, hs, mask_id):
    """The two-kernel build of the comparison library (a metadata kernel, then
    a copy of the hidden rows through a row map) on the same inputs as
    peagle_build_draft_batch: returns (call, outputs)."""
    import ctypes
    vp, i = ctypes.c_void_p, ctypes.c_int
    fn = _ceiling_fn("svc_build_split", [vp] * 5 + [i, i, vp, vp, ctypes.c_int32, i, i, i]
                     + [vp] * 7)
    B, K = d.shape
    H = hid.shape[1]
    dev = d.device
    outs = {"input_ids": torch.empty(B * 2 * K, dtype=torch.int32, device=dev),
            "positions": torch.empty(B * 2 * K, dtype=torch.int64, device=dev),
            "slot_mapping": torch.empty(B * 2 * K, dtype=torch.int64, device=dev),
            "hidden": torch.empty((B * 2 * K, H), dtype=hid.dtype, device=dev),
            "sample_rows": torch.empty((B, K), dtype=torch.int32, device=dev)}
    maps = torch.empty(2 * B * (K + 1), dtype=torch.int32, device=dev)

    def call():
        if fn(o.data_ptr(), a.data_ptr(), d.data_ptr(), L.data_ptr(), bt.data_ptr(), bt.shape[1],
              block_size, hid.data_ptr(), hs.data_ptr(), mask_id, B, K, H,
              outs["input_ids"].data_ptr(), outs["positions"].data_ptr(),
              outs["slot_mapping"].data_ptr(), outs["hidden"].data_ptr(),
              outs["sample_rows"].data_ptr(), maps.data_ptr(),
              torch.cuda.current_stream().cuda_stream):
            raise RuntimeError("svc_build_split failed")
    return call, outs


def build_compare(torch, build, bouts, split_call, souts):
    """GPU time per call of the fused build and the two-kernel build, and
    whether their outputs are bit for bit the same."""
    build()
    split_call()
    torch.cuda.synchronize()
    same = all(torch.equal(bouts[k].view(torch.int16) if bouts[k].dtype == torch.bfloat16
                           else bouts[k],
                           souts[k].view(torch.int16) if souts[k].dtype == torch.bfloat16
                           else souts[k]) for k in souts)
    return {"fused_gpu_us_per_call": gpu_us_per_call(torch, build),
            "two_kernels_gpu_us_per_call": gpu_us_per_call(torch, split_call),
            "same_outputs": same}


def read_ceiling(torch, buf, reps):
    """The read rate of a plain streaming kernel over the same resident device
    buffer (8192 workgroups, 8 16-byte loads in flight per lane, nothing
    stored), with non-temporal and with cached loads: the practical ceiling
    the row kernel is held against, beside the nominal peak."""
    fn = _stream_read_fn()
    nbytes = buf.numel() * buf.element_size()
    stream = torch.cuda.current_stream()
    out = {"bytes": nbytes,
           "kernel": "plain streaming read: 8192 workgroups x 256 threads, 8 x 16-byte loads "
                     "in flight per thread, one pass over the logit buffer"}
    for nt, key in ((1, "nontemporal_gbs"), (0, "cached_gbs")):
        for _ in range(3):
            if fn(buf.data_ptr(), nbytes, nt, stream.cuda_stream):
                raise RuntimeError("svc_stream_read failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn(buf.data_ptr(), nbytes, nt, stream.cuda_stream)
        e1.record(stream)
        e1.synchronize()
        out[key] = nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    return out


def graph_bench(sv, torch, np, args, B, K, V, vi, bi, z, q, d, u, L, bt, hid, hs, out_t, acc_t,
                pd_t, ws, bouts):
    """The fused sampled step (verify, build, acceptance metrics) replayed as
    one captured HIP graph vs the same calls launched one by one, at the full
    batch and at small batches (the first 16 sequences, the first one) where
    launches and the kernels' own latency dominate; the metrics counters give
    the acceptance figures."""
    def run(nb):
        zz, qq, dd, uu = z[:nb], q[:nb], d[:nb], u[:nb]
        oo = {k: (v[:nb * 2 * K] if k != "sample_rows" else v[:nb]) for k, v in bouts.items()}
        m_e, m_g = sv.accept_metrics_buffer(K, z.device), sv.accept_metrics_buffer(K, z.device)
        build = dict(start_pos=L[:nb], block_table=bt[:nb], block_size=bi.spec.block_size,
                     target_hidden=hid[:nb * (K + 1)], h_shared=hs,
                     mask_token_id=bi.mask_token_id, outputs=oo)

        def eager():
            sv.spec_verify_sample(zz, qq, dd, uu, vi.temperature, out_tokens=out_t[:nb],
                                  out_num_accepted=acc_t[:nb], out_draft_target_prob=pd_t[:nb],
                                  workspace=ws)
            sv.peagle_build_draft_batch(out_t[:nb], acc_t[:nb], dd, build["start_pos"],
                                        build["block_table"], build["block_size"],
                                        build["target_hidden"], hs, bi.mask_token_id, outputs=oo)
            sv.spec_accept_metrics(acc_t[:nb], K, m_e)

        g = sv.StepGraph("sample", dict(target_logits=zz, draft_probs=qq, draft_tokens=dd,
                                        uniforms=uu, temperature=vi.temperature,
                                        out_tokens=out_t[:nb], out_num_accepted=acc_t[:nb],
                                        out_draft_target_prob=pd_t[:nb], workspace=ws),
                         build, metrics=m_g)
        out = {"B": nb}
        for name, fn in (("eager", eager), ("graph", g.launch)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            with quiet_host():
                t0 = time.perf_counter()
                for _ in range(args.steps):
                    fn()
                torch.cuda.synchronize()
                out[f"{name}_ms_per_step"] = (time.perf_counter() - t0) / args.steps * 1e3
        g.close()
        summ = sv.acceptance_summary(m_g)
        out["rows_per_s_graph"] = nb * (K + 1) / (out["graph_ms_per_step"] * 1e-3)
        out["device_metrics"] = {k: summ[k] for k in ("steps", "acceptance_length",
                                                      "tokens_per_round",
                                                      "draft_acceptance_rate")}
        return out
    return {"note": "verify_sample + P-EAGLE build + acceptance metrics per step",
            "full": run(B), "small": run(16), "single": run(1)}


def early_exit_bench(sv, torch, np, args, B, K, V, vi, bi, z, q, d, u, temps, L, bt, hid, hs,
                     ws, bouts):
    """The fused step with the early-exit verify forms against the full ones
    (each + P-EAGLE build, same inputs): wall time per step, the row
    statistics launches, the logit rows read, and whether tokens and accept
    counts are identical.  Not the headline figure: these forms skip the rows
    past each sequence's first rejection."""
    dev = z.device
    T = vi.temperature
    outs = {}
    res = {"workload": f"B={B} K={K} V={V} bf16 + P-EAGLE build H={hid.shape[1]}; the early-exit "
                       "forms read only the rows up to each sequence's first rejection "
                       "(draft positions in launch ranges [0,1), [1,2), [2,4), [4,8))"}
    calls = {
        "greedy": (sv.spec_verify_greedy, sv.spec_verify_greedy_early_exit, (z, d), {}),
        "sample": (sv.spec_verify_sample, sv.spec_verify_sample_early_exit, (z, q, d, u, T), {}),
        "mixed": (sv.spec_verify_mixed, sv.spec_verify_mixed_early_exit, (z, q, d, u, temps), {}),
    }
    for mode, (full, ee, a, kw) in calls.items():
        for name, fn in (("full", full), ("early_exit", ee)):
            ot = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
            oa = torch.empty((B,), dtype=torch.int32, device=dev)

            def step():
                fn(*a, out_tokens=ot, out_num_accepted=oa, workspace=ws)
                sv.peagle_build_draft_batch(ot, oa, d, L, bt, bi.spec.block_size, hid, hs,
                                            bi.mask_token_id, outputs=bouts)
            ms = wall_ms(torch, step, args.warmup, args.steps)
            sv.trace_begin(64)
            step()
            torch.cuda.synchronize()
            kern = [(k, m) for k, m in sv.trace_read()]
            sv.trace_end()
            rows_launches = [m for k, m in kern if k.endswith("_rows")]
            outs[(mode, name)] = (ot.clone(), oa.clone())
            res[f"{mode}_{name}_ms_per_step"] = ms
            res[f"{mode}_{name}_rows_launch_ms"] = rows_launches
        acc = outs[(mode, "full")][1].long()
        res[f"{mode}_rows_needed"] = int((acc + 1).clamp(max=K + 1).sum().item())
        res[f"{mode}_speedup"] = (res[f"{mode}_full_ms_per_step"]
                                  / res[f"{mode}_early_exit_ms_per_step"])
        res[f"{mode}_identical_outputs"] = bool(
            torch.equal(outs[(mode, "full")][0], outs[(mode, "early_exit")][0])
            and torch.equal(outs[(mode, "full")][1], outs[(mode, "early_exit")][1]))
    res["rows_total"] = B * (K + 1)
    return res


def round_bench(sv, torch, np, args, B, K, V, vi, bi, z, d, u, L, bt, hid, hs, out_t, acc_t,
                pd_t, ws, bouts, temps):
    """One decode round of the path on the two ways of handing the drafter's
    distributions to the verify: drafter sampling that writes dense fp32 q +
    spec_verify_sample, vs drafter sampling that writes only tokens and row
    descriptors + spec_verify_sample_lq; both followed by the P-EAGLE build.
    Stand-in drafter rows: the first K logit rows of the sequence B/2 places
    away (same recipe, distinct memory), gathered through a row index.  The
    same pair is also timed on a mixed serving batch (per-sequence
    temperatures, each sequence's drafter rows sampled at its own
    temperature): spec_verify_mixed vs spec_verify_mixed_lq.  One more
    round pairs the drafter-logit interface with the early-exit verify."""
    dev = z.device
    zr = z.view(B * (K + 1), V)
    seq = (torch.arange(B, dtype=torch.int32, device=dev) + B // 2) % B
    rows = (seq[:, None] * (K + 1) + torch.arange(K, dtype=torch.int32, device=dev)[None, :]).contiguous()
    ud = torch.from_numpy(np.random.default_rng(8).random((B, K), dtype=np.float32)).to(dev)
    tok = torch.empty((B, K), dtype=torch.int32, device=dev)
    q = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    desc = torch.empty((B, K, 4), dtype=torch.int32, device=dev)
    T = vi.temperature

    def build():
        sv.peagle_build_draft_batch(out_t, acc_t, tok, L, bt, bi.spec.block_size, hid, hs,
                                    bi.mask_token_id, outputs=bouts)

    def dense():
        sv.spec_draft_sample(zr, K, T, uniforms=ud, row_index=rows, out_draft_tokens=tok,
                             out_draft_probs=q)
        sv.spec_verify_sample(z, q, tok, u, T, out_tokens=out_t, out_num_accepted=acc_t,
                              out_draft_target_prob=pd_t, workspace=ws)
        build()

    def lq():
        sv.spec_draft_sample(zr, K, T, uniforms=ud, row_index=rows, out_draft_tokens=tok,
                             want_draft_probs=False, out_row_desc=desc)
        sv.spec_verify_sample_lq(z, zr, desc, tok, u, T, drafter_rows=rows, out_tokens=out_t,
                                 out_num_accepted=acc_t, out_draft_target_prob=pd_t, workspace=ws)
        build()

    def lq_ee():
        sv.spec_draft_sample(zr, K, T, uniforms=ud, row_index=rows, out_draft_tokens=tok,
                             want_draft_probs=False, out_row_desc=desc)
        sv.spec_verify_sample_lq_early_exit(z, zr, desc, tok, u, T, drafter_rows=rows,
                                            out_tokens=out_t, out_num_accepted=acc_t,
                                            out_draft_target_prob=pd_t, workspace=ws)
        build()

    def dense_mixed():
        sv.spec_draft_sample(zr, K, T, uniforms=ud, row_index=rows, temperatures=temps,
                             out_draft_tokens=tok, out_draft_probs=q)
        sv.spec_verify_mixed(z, q, tok, u, temps, out_tokens=out_t, out_num_accepted=acc_t,
                             out_draft_target_prob=pd_t, workspace=ws)
        build()

    def lq_mixed():
        sv.spec_draft_sample(zr, K, T, uniforms=ud, row_index=rows, temperatures=temps,
                             out_draft_tokens=tok, want_draft_probs=False, out_row_desc=desc)
        sv.spec_verify_mixed_lq(z, zr, desc, tok, u, temps, drafter_rows=rows, out_tokens=out_t,
                                out_num_accepted=acc_t, out_draft_target_prob=pd_t, workspace=ws)
        build()

    res = {"workload": f"B={B} K={K} V={V} bf16: drafter sampling + sampled verify + P-EAGLE build"}
    outs = {}
    for name, fn in (("dense_q", dense), ("logit_q", lq), ("logit_q_early_exit", lq_ee),
                     ("mixed_dense_q", dense_mixed), ("mixed_logit_q", lq_mixed)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        with quiet_host():
            t0 = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            res[f"{name}_ms_per_round"] = (time.perf_counter() - t0) / args.steps * 1e3
        outs[name] = (out_t.clone(), acc_t.clone())
    res["speedup"] = res["dense_q_ms_per_round"] / res["logit_q_ms_per_round"]
    res["identical_outputs"] = bool(torch.equal(outs["dense_q"][0], outs["logit_q"][0]) and
                                    torch.equal(outs["dense_q"][1], outs["logit_q"][1]))
    res["early_exit_identical_outputs"] = bool(
        torch.equal(outs["dense_q"][0], outs["logit_q_early_exit"][0]) and
        torch.equal(outs["dense_q"][1], outs["logit_q_early_exit"][1]))
    res["mixed_speedup"] = res["mixed_dense_q_ms_per_round"] / res["mixed_logit_q_ms_per_round"]
    res["mixed_identical_outputs"] = bool(
        torch.equal(outs["mixed_dense_q"][0], outs["mixed_logit_q"][0]) and
        torch.equal(outs["mixed_dense_q"][1], outs["mixed_logit_q"][1]))
    return res


def percentiles(np, xs):
    """p10 / p50 / p90 of a list of times (ms)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90))}


def wall_ms(torch, call, warmup, steps):
    """Wall time per call (ms) of `steps` calls after `warmup` untimed ones."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    with quiet_host():
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3


def kernel_times(sv, torch, np, call, steps):
    """Average duration (ms) of each kernel that `call` launches, every kernel
    timed in a loop of its own with only it traced (two events per call)."""
    sv.trace_begin(16)
    call()
    torch.cuda.synchronize()
    names = list(dict.fromkeys(name for name, _ in sv.trace_read()))
    sv.trace_end()
    out = {}
    for name in names:
        sv.trace_begin(4 * steps, [name])
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        out[name] = float(np.mean([ms for _, ms in sv.trace_read()]))
        sv.trace_end()
    return out


def gpu_us_per_call(torch, call, n=100, reps=5):
    """The GPU's own time per call: n calls captured in one graph (the
    library enqueues on torch's current stream, the capture stream), replayed
    reps times; no host work between the calls."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            call()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    e1.synchronize()
    us = e0.elapsed_time(e1) / (reps * n) * 1e3
    del g
    return us


def small_workloads_bench(sv, torch, np, synth, args):
    """The smaller workloads, each on its own: the tiny verify (B=1, K=3,
    V=32 fp32: launch latency), the mid-size verify (B=8, K=5, V=32000 fp32,
    T=1: 48 logit rows, bound by latency), the P-EAGLE build (B=64, K=7,
    H=2880 bf16: 8 MB of data movement), and the large-vocabulary verify
    (B=64, K=7, V=201088 bf16, T=0.7: 206 MB of logits, under the 256 MB
    Infinity Cache, so the calls rotate over four copies of the logits and
    draft probabilities; the same calls on one resident copy are timed too).
    Per call: the host-loop wall time, the GPU's own time (calls captured in
    one graph), each kernel's duration, and the algorithmic bytes over the
    kernels' time."""
    dev = torch.device("cuda:0")
    steps = max(args.steps, 100)

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    def entry(call, nbytes):
        ms = wall_ms(torch, call, args.warmup, steps)
        kms = kernel_times(sv, torch, np, call, steps)
        gpu_ms = sum(kms.values())
        return {"ms_per_call": ms, "kernels_ms": kms, "algorithmic_bytes": nbytes,
                "gbs_over_kernel_time": nbytes / (gpu_ms * 1e-3) / 1e9,
                "frac_over_kernel_time": nbytes / (gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    res = {}
    for n, copies in ((1, 1), (2, 1), (4, 4)):
        vi = synth.make_verify_inputs(synth.verify_config(n), workers=args.workers)
        B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
        zsize = 2 if vi.spec.dtype == "bf16" else 4
        zs = [up(vi.logits)]
        qs = [up(vi.draft_probs)]
        for _ in range(copies - 1):
            zs.append(zs[0].clone())
            qs.append(qs[0].clone())
        d, u = up(vi.draft_tokens), up(vi.uniforms)
        out_t = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        acc_t = torch.empty(B, dtype=torch.int32, device=dev)
        pd_t = torch.empty((B, K), dtype=torch.float32, device=dev)
        ws = torch.zeros(sv.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
        turn = [0]

        def sample():
            i = turn[0] = (turn[0] + 1) % copies
            sv.spec_verify_sample(zs[i], qs[i], d, u, vi.temperature, out_tokens=out_t,
                                  out_num_accepted=acc_t, out_draft_target_prob=pd_t,
                                  workspace=ws)

        def greedy():
            i = turn[0] = (turn[0] + 1) % copies
            sv.spec_verify_greedy(zs[i], d, out_tokens=out_t, out_num_accepted=acc_t,
                                  workspace=ws)

        r = {"workload": f"{synth.CONFIG_NAMES[n]}: B={B} K={K} V={V} {vi.spec.dtype} logits, "
                         f"T={vi.temperature}" + (f"; {copies} rotating input copies" if
                                                  copies > 1 else "")}
        for name, fn, smp in (("sample", sample, True), ("greedy", greedy, False)):
            fn()
            torch.cuda.synchronize()
            rb, sb = verify_bytes(B, K, V, zsize, acc_t.cpu().numpy(), sample=smp)
            r[name] = entry(fn, rb + sb)
            r[name]["gpu_us_per_call"] = gpu_us_per_call(torch, fn)

        # the early-exit forms (row statistics only up to each sequence's
        # first rejection): GPU time per call, to show where they pay
        def sample_ee():
            i = turn[0] = (turn[0] + 1) % copies
            sv.spec_verify_sample_early_exit(zs[i], qs[i], d, u, vi.temperature,
                                             out_tokens=out_t, out_num_accepted=acc_t,
                                             out_draft_target_prob=pd_t, workspace=ws)

        def greedy_ee():
            i = turn[0] = (turn[0] + 1) % copies
            sv.spec_verify_greedy_early_exit(zs[i], d, out_tokens=out_t, out_num_accepted=acc_t,
                                             workspace=ws)
        r["early_exit_gpu_us_per_call"] = {"sample": gpu_us_per_call(torch, sample_ee),
                                           "greedy": gpu_us_per_call(torch, greedy_ee)}
        if copies > 1:
            # the same calls on one resident copy: the Infinity Cache then
            # holds all 206 MB of logits between calls
            def one_copy():
                sv.spec_verify_sample(zs[0], qs[0], d, u, vi.temperature, out_tokens=out_t,
                                      out_num_accepted=acc_t, out_draft_target_prob=pd_t,
                                      workspace=ws)
            r["sample_one_resident_copy"] = {
                "ms_per_call": wall_ms(torch, one_copy, args.warmup, steps),
                "kernels_ms": kernel_times(sv, torch, np, one_copy, steps),
                "gpu_us_per_call": gpu_us_per_call(torch, one_copy)}
        if copies == 1:
            g = sv.StepGraph("sample", dict(target_logits=zs[0], draft_probs=qs[0],
                                            draft_tokens=d, uniforms=u,
                                            temperature=vi.temperature, out_tokens=out_t,
                                            out_num_accepted=acc_t, out_draft_target_prob=pd_t,
                                            workspace=ws))
            r["sample"]["graph_ms_per_call"] = wall_ms(torch, g.launch, args.warmup, steps)
            g.close()
            g = sv.StepGraph("greedy", dict(target_logits=zs[0], draft_tokens=d, out_tokens=out_t,
                                            out_num_accepted=acc_t, workspace=ws))
            r["greedy"]["graph_ms_per_call"] = wall_ms(torch, g.launch, args.warmup, steps)
            g.close()
        res[synth.CONFIG_NAMES[n]] = r
        del zs, qs
    bi = synth.make_build_inputs(synth.build_config(3))
    B, K, H = bi.spec.B, bi.spec.K, bi.spec.H
    o, a, d = up(bi.out_tokens), up(bi.num_accepted), up(bi.draft_tokens)
    L, bt, hid, hs = up(bi.start_pos), up(bi.block_table), up(bi.target_hidden), up(bi.h_shared)
    bouts = sv.peagle_build_draft_batch(o, a, d, L, bt, bi.spec.block_size, hid, hs,
                                        bi.mask_token_id)

    def build():
        sv.peagle_build_draft_batch(o, a, d, L, bt, bi.spec.block_size, hid, hs,
                                    bi.mask_token_id, outputs=bouts)

    res[synth.CONFIG_NAMES[3]] = {"workload": f"{synth.CONFIG_NAMES[3]}: B={B} K={K} H={H} bf16",
                                  "build": entry(build, build_bytes(B, K, H, 2))}
    res[synth.CONFIG_NAMES[3]]["build"]["gpu_us_per_call"] = gpu_us_per_call(torch, build)
    scall, souts = split_build(torch, o, a, d, L, bt, bi.spec.block_size, hid, hs,
                               bi.mask_token_id)
    res[synth.CONFIG_NAMES[3]]["build_vs_two_kernels"] = build_compare(torch, build, bouts, scall,
                                                                       souts)
    return res


def fp32_bench(sv, torch, np, args, vi, z, q, d, u, ws):
    """The B=1024 K=7 V=151936 verify with its logits widened to fp32 (the same values,
    4.98 GB): engines often hand the sampler fp32 logits."""
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    z32 = z.float()
    out_t = torch.empty((B, K + 1), dtype=torch.int32, device=z.device)
    acc_t = torch.empty(B, dtype=torch.int32, device=z.device)
    res = {"workload": f"B={B} K={K} V={V} fp32 logits (the bf16 batch widened), "
                       f"T={vi.temperature}"}

    def sample():
        sv.spec_verify_sample(z32, q, d, u, vi.temperature, out_tokens=out_t,
                              out_num_accepted=acc_t, workspace=ws)

    def greedy():
        sv.spec_verify_greedy(z32, d, out_tokens=out_t, out_num_accepted=acc_t, workspace=ws)

    for name, fn, smp, rows_k in (("sample", sample, True, "verify_sample_rows"),
                                  ("greedy", greedy, False, "verify_greedy_rows")):
        ms = wall_ms(torch, fn, args.warmup, args.steps)
        kms = kernel_times(sv, torch, np, fn, args.steps)
        rb, sb = verify_bytes(B, K, V, 4, acc_t.cpu().numpy(), sample=smp)
        rk = kms[rows_k]
        res[name] = {"ms_per_call": ms, "kernels_ms": kms, "algorithmic_bytes": rb + sb,
                     "call_gbs": (rb + sb) / (ms * 1e-3) / 1e9,
                     "rows_gbs": rb / (rk * 1e-3) / 1e9,
                     "rows_frac": rb / (rk * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del z32
    return res


def tree_walk_passes(np, parents, path, num_accepted):
    """Row passes of the sampled tree walk, counted from its outputs.  At each
    node on the accepted path the walk tests the node's children in index
    order; every rejected child costs one workgroup pass over the node's logit
    and draft-probability rows (the new residual's mass).  At the last node
    every child was rejected; a node with no children costs one pass over its
    logit row alone (the target distribution's tile masses for the final
    draw).  Returns per tree (residual passes, logit-only passes).  (A
    residual that rounds to zero mass adds one logit-only pass; it is not
    counted here.)"""
    B, N = parents.shape
    res = np.zeros(B, np.int64)
    plain = np.zeros(B, np.int64)
    for b in range(B):
        a = int(num_accepted[b])
        cur = 0
        for depth in range(a + 1):
            kids = [i for i in range(1, N + 1) if int(parents[b, i - 1]) == cur]
            if depth < a:
                nxt = int(path[b, depth])
                res[b] += sum(1 for i in kids if i < nxt)
                cur = nxt
            elif kids:
                res[b] += len(kids)
            else:
                plain[b] += 1
    return res, plain


def tree_bench(sv, torch, np, synth, args):
    """Draft-tree verification on B=256 trees of 15 nodes (3 children at the
    root, 2 below each, 1 below those), V=151936 bf16 logits, T=0.7: one call
    is the row statistics of all B*16 rows plus the walk down every tree."""
    spec = synth.TREE_CONFIGS["tree-bench"]
    ti = synth.make_tree_inputs(spec, workers=args.workers)
    dev = torch.device("cuda:0")

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    z, q, par, tok, u = (up(ti.logits), up(ti.draft_probs), up(ti.parents), up(ti.tokens),
                         up(ti.uniforms))
    B, N, V = spec.B, spec.N, spec.V
    ws = torch.zeros(sv.spec_verify_workspace_bytes(B, N, V), dtype=torch.uint8, device=dev)
    outs = (torch.empty((B, N + 1), dtype=torch.int32, device=dev),
            torch.empty((B, N + 1), dtype=torch.int32, device=dev),
            torch.empty(B, dtype=torch.int32, device=dev))
    rows = B * (N + 1)
    res = {"workload": f"B={B} trees of N={N} nodes (widths 3,2,1), V={V} bf16, T={spec.temperature}"}
    for name, T in (("greedy", 0.0), ("sample", spec.temperature)):
        def call():
            sv.spec_verify_tree(z, par, tok, T, draft_probs=q, uniforms=u, out_tokens=outs[0],
                                out_path=outs[1], out_num_accepted=outs[2], workspace=ws)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        with quiet_host():
            t0 = time.perf_counter()
            for _ in range(args.steps):
                call()
            torch.cuda.synchronize()
            sec = (time.perf_counter() - t0) / args.steps
        sv.trace_begin(4 * args.steps)
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        per = {}
        for k, ms in sv.trace_read():
            per.setdefault(k, []).append(ms)
        sv.trace_end()
        acc = outs[2].cpu().numpy()
        rb = rows * V * 2
        kms = {k: float(np.mean(v)) for k, v in per.items()}
        res[name] = {"ms_per_call": sec * 1e3, "rows_per_s": rows / sec,
                     "logit_gbs": rb / sec / 1e9, "logit_frac": rb / sec / 1e9 / HBM_PEAK_GBS,
                     "kernels_ms": kms, "mean_accepted": float(acc.mean())}
        if T > 0.0:
            # what the walk's row passes read (each pass re-reads the node's
            # logit row, and its fp32 draft row after a rejection)
            rp, pp = tree_walk_passes(np, ti.parents, outs[1].cpu().numpy(), acc)
            wb = int(rp.sum()) * V * (2 + 4) + int(pp.sum()) * V * 2
            walk_ms = kms.get("tree_walk")
            passes = rp + pp
            res[name]["walk"] = {
                "passes_mean": float(passes.mean()), "passes_max": int(passes.max()),
                "pass_bytes": wb,
                "pass_gbs": wb / (walk_ms * 1e-3) / 1e9 if walk_ms else None,
                "note": "bytes read by the walk's workgroup passes (a node's logit row, plus "
                        "its fp32 draft row after a rejection); one workgroup per tree, so "
                        "the walk lasts as long as the tree with the most passes"}
        # the early-exit form: no row kernel, the walk computes the statistics
        # of the rows it visits (same inputs, same definitions)
        ref = [x.clone() for x in outs]

        def call_ee():
            sv.spec_verify_tree_early_exit(z, par, tok, T, draft_probs=q, uniforms=u,
                                           out_tokens=outs[0], out_path=outs[1],
                                           out_num_accepted=outs[2], workspace=ws)
        ee_ms = wall_ms(torch, call_ee, args.warmup, args.steps)
        same = sum(bool(torch.equal(outs[0][b], ref[0][b]) and torch.equal(outs[1][b], ref[1][b]))
                   for b in range(B))
        res[name]["early_exit"] = {
            "ms_per_call": ee_ms, "speedup": sec * 1e3 / ee_ms, "trees_identical": same,
            "rows_visited": int(outs[2].long().sum().item()) + B}
    # a mixed serving batch of trees: per-tree temperatures from {0, 0.5, 0.7,
    # 1.0, 1.3}, full and early-exit forms
    temps_np = synth.make_temperatures(B, 62)
    temps = up(temps_np)
    res["mixed"] = {"greedy_trees": int((temps_np == 0).sum()), "sampled_trees": int(
        (temps_np > 0).sum())}
    for name, fn in (("full", sv.spec_verify_tree_mixed),
                     ("early_exit", sv.spec_verify_tree_mixed_early_exit)):
        def call_m():
            fn(z, par, tok, temps, q, u, out_tokens=outs[0], out_path=outs[1],
               out_num_accepted=outs[2], workspace=ws)
        res["mixed"][f"{name}_ms_per_call"] = wall_ms(torch, call_m, args.warmup, args.steps)
    res["drafter_logits"] = tree_lq_bench(sv, torch, np, args, spec, z, par, tok, u, ws, outs)
    return res


def tree_lq_bench(sv, torch, np, args, spec, z, par, tok, u, ws, outs):
    """The sampled tree call with the drafter's distributions handed over two
    ways, on one drafting: stand-in drafter rows (the tree's target rows plus
    seeded N(0, 1) noise, bf16, one per node) sampled at T=0.7 by
    spec_draft_sample, which writes the dense q and the row descriptors; then
    spec_verify_tree on the dense q and spec_verify_tree_lq on the drafter
    logits + descriptors (identical outputs).  `round` adds the drafting each
    way needs: the drafter kernel writing dense q, or only tokens and row
    descriptors."""
    B, N, V = spec.B, spec.N, spec.V
    n = B * (N + 1)
    dev = z.device
    g = torch.Generator(device=dev)
    g.manual_seed(41)
    zd = (z.view(n, V).float() + torch.randn((n, V), generator=g, device=dev)).to(z.dtype)
    ud = torch.rand((n, 1), generator=g, device=dev)
    _, q, desc = sv.spec_draft_sample(zd, 1, spec.temperature, uniforms=ud, want_row_desc=True)
    q, desc = q.view(B, N + 1, V), desc.view(B, N + 1, 4)
    T = spec.temperature
    lq_outs = tuple(torch.empty_like(x) for x in outs)
    calls = {
        "dense_q": lambda: sv.spec_verify_tree(z, par, tok, T, draft_probs=q, uniforms=u,
                                               out_tokens=outs[0], out_path=outs[1],
                                               out_num_accepted=outs[2], workspace=ws),
        "logit_q": lambda: sv.spec_verify_tree_lq(z, zd, desc, par, tok, u, T,
                                                  out_tokens=lq_outs[0], out_path=lq_outs[1],
                                                  out_num_accepted=lq_outs[2], workspace=ws)}
    res = {"workload": f"B={B} trees of N={N} nodes, V={V} bf16, T={T}; drafter rows = target "
                       "rows + N(0,1) noise, drafted at T=0.7"}
    for name, call in calls.items():
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        with quiet_host():
            t0 = time.perf_counter()
            for _ in range(args.steps):
                call()
            torch.cuda.synchronize()
            sec = (time.perf_counter() - t0) / args.steps
        sv.trace_begin(4 * args.steps)
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        per = {}
        for k, ms in sv.trace_read():
            per.setdefault(k, []).append(ms)
        sv.trace_end()
        res[name] = {"ms_per_call": sec * 1e3,
                     "kernels_ms": {k: float(np.mean(v)) for k, v in per.items()}}
    res["identical_outputs"] = all(torch.equal(a, b) for a, b in zip(outs, lq_outs))
    dtok = torch.empty((n, 1), dtype=torch.int32, device=dev)
    drafts = {
        "dense_q": lambda: sv.spec_draft_sample(zd, 1, T, uniforms=ud, out_draft_tokens=dtok,
                                                out_draft_probs=q.view(n, 1, V)),
        "logit_q": lambda: sv.spec_draft_sample(zd, 1, T, uniforms=ud, out_draft_tokens=dtok,
                                                want_draft_probs=False,
                                                out_row_desc=desc.view(n, 1, 4))}
    for name, call in drafts.items():
        res[name]["drafter_ms"] = wall_ms(torch, call, args.warmup, args.steps)
        res[name]["round_ms"] = res[name]["drafter_ms"] + res[name]["ms_per_call"]
    acc = outs[2].cpu().numpy()
    rp, pp = tree_walk_passes(np, par.cpu().numpy(), outs[1].cpu().numpy(), acc)
    res["mean_accepted"] = float(acc.mean())
    res["passes_mean"] = float((rp + pp).mean())
    res["passes_max"] = int((rp + pp).max())
    # bytes of the walk's passes: a node's logit row, plus after a rejection
    # its fp32 q row (dense) or its bf16 drafter logit row (logit q)
    res["dense_q"]["pass_bytes"] = int(rp.sum()) * V * (2 + 4) + int(pp.sum()) * V * 2
    res["logit_q"]["pass_bytes"] = int(rp.sum()) * V * (2 + 2) + int(pp.sum()) * V * 2
    return res


def profile_large_vocab(args, np, synth, log):
    """For the profiler: the large-vocabulary verify (B=64 K=7 V=201088 bf16,
    T=0.7), sampled and greedy, rotating over four copies of its inputs as the
    bench times it (args.profile_steps rounds of four calls each), then the
    read-ceiling kernel over one logit copy and the 1 GiB counter-calibration
    copy."""
    log("drawing the large-vocabulary inputs")
    vi = synth.make_verify_inputs(synth.verify_config(4), workers=1)
    import torch
    import draft_verification_vocab_amd as sv
    sv.require_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    zs = [up(vi.logits) for _ in range(4)]
    qs = [up(vi.draft_probs) for _ in range(4)]
    d, u = up(vi.draft_tokens), up(vi.uniforms)
    for i in range(args.profile_steps * 4):
        sv.spec_verify_sample(zs[i % 4], qs[i % 4], d, u, vi.temperature)
    for i in range(args.profile_steps * 4):
        sv.spec_verify_greedy(zs[i % 4], d)
    torch.cuda.synchronize()
    rd = _stream_read_fn()
    if rd(zs[0].data_ptr(), zs[0].numel() * zs[0].element_size(), 1,
          torch.cuda.current_stream().cuda_stream):
        raise RuntimeError("svc_stream_read failed")
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    if args.hash_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.hash_out)), exist_ok=True)
        with open(args.hash_out, "w") as f:
            f.write(kernel_source_hash() + " large-vocab\n")
    print(f"profiled {args.profile_steps} rounds of the large-vocabulary verify, the read-ceiling "
          "kernel and a 1 GiB copy", flush=True)


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.ingest_valu:
        ingest_valu(args.ingest_valu)
        return
    if args.ingest_trace:
        ingest_trace(*args.ingest_trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import synth

    # inputs are drawn before anything touches the GPU
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    if args.profile_steps and args.profile_workload == "large-vocab":
        profile_large_vocab(args, np, synth, log)
        return
    log("drawing inputs")
    workers = 1 if args.profile_steps else args.workers
    vi, bi = synth.make_fused_inputs(workers=workers)
    cpu_all = None
    if args.cpu_budget > 0 and not args.profile_steps:
        # before the GPU is touched: forked workers share the inputs
        log("timing the CPU oracle on all cores")
        cpu_all = cpu_baseline_all_cores(vi, bi, min(16, os.cpu_count() or 1))
    log("inputs ready; uploading")
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    H = bi.spec.H

    import torch
    import draft_verification_vocab_amd as sv
    sv.require_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    z, q, d, u = up(vi.logits), up(vi.draft_probs), up(vi.draft_tokens), up(vi.uniforms)
    L, bt, hid, hs = up(bi.start_pos), up(bi.block_table), up(bi.target_hidden), up(bi.h_shared)
    out_t = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    acc_t = torch.empty(B, dtype=torch.int32, device=dev)
    pd_t = torch.empty((B, K), dtype=torch.float32, device=dev)
    ws = torch.zeros(sv.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
    bouts = {"input_ids": torch.empty(B * 2 * K, dtype=torch.int32, device=dev),
             "positions": torch.empty(B * 2 * K, dtype=torch.int64, device=dev),
             "slot_mapping": torch.empty(B * 2 * K, dtype=torch.int64, device=dev),
             "hidden": torch.empty((B * 2 * K, H), dtype=torch.bfloat16, device=dev),
             "sample_rows": torch.empty((B, K), dtype=torch.int32, device=dev)}

    # drafter-output sampling: K prediction rows per sequence.  The synthetic
    # drafter rows are the first K logit rows of each sequence (same recipe:
    # bf16, 3*N(0,1) + Zipf head), gathered through a row index as the drafter
    # batch's sample_rows would be.
    d_rows = (torch.arange(B, dtype=torch.int32, device=dev)[:, None] * (K + 1)
              + torch.arange(K, dtype=torch.int32, device=dev)[None, :]).contiguous()
    d_u = up(np.random.default_rng(7).random((B, K), dtype=np.float32))
    d_tok = torch.empty((B, K), dtype=torch.int32, device=dev)
    d_q = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    z_rows = z.view(B * (K + 1), V)

    def draft(with_q=True):
        sv.spec_draft_sample(z_rows, K, vi.temperature, uniforms=d_u, row_index=d_rows,
                             out_draft_tokens=d_tok, out_draft_probs=d_q if with_q else None,
                             want_draft_probs=with_q)

    # a mixed serving batch: per-sequence temperatures from {0, 0.5, 0.7, 1.0, 1.3}
    temps_np = synth.make_temperatures(B, 15)
    temps = up(temps_np)

    def step(sample=True):
        if sample == "mixed":
            sv.spec_verify_mixed(z, q, d, u, temps, out_tokens=out_t, out_num_accepted=acc_t,
                                 out_draft_target_prob=pd_t, workspace=ws)
        elif sample:
            sv.spec_verify_sample(z, q, d, u, vi.temperature, out_tokens=out_t,
                                  out_num_accepted=acc_t, out_draft_target_prob=pd_t, workspace=ws)
        else:
            sv.spec_verify_greedy(z, d, out_tokens=out_t, out_num_accepted=acc_t, workspace=ws)

    def build():
        sv.peagle_build_draft_batch(out_t, acc_t, d, L, bt, bi.spec.block_size, hid, hs,
                                    bi.mask_token_id, outputs=bouts)

    if args.profile_steps:
        # every kernel family once per step, for the profiler: sampled, greedy
        # and mixed verify with the build, drafter sampling with q and with
        # row descriptors, the verify from drafter logits (uniform and mixed
        # temperatures), the early-exit sampled and greedy verify, acceptance
        # metrics, and (below) tree verification
        d_desc = torch.empty((B, K, 4), dtype=torch.int32, device=dev)
        m_desc = torch.empty((B, K, 4), dtype=torch.int32, device=dev)
        mtr = sv.accept_metrics_buffer(K, dev)
        for i in range(args.profile_steps):
            step(True); build(); step(False); build(); step("mixed"); build(); draft()
            sv.spec_draft_sample(z_rows, K, vi.temperature, uniforms=d_u, row_index=d_rows,
                                 out_draft_tokens=d_tok, want_draft_probs=False,
                                 out_row_desc=d_desc)
            sv.spec_verify_sample_lq(z, z_rows, d_desc, d_tok, u, vi.temperature,
                                     drafter_rows=d_rows, out_tokens=out_t,
                                     out_num_accepted=acc_t, workspace=ws)
            sv.spec_draft_sample(z_rows, K, vi.temperature, uniforms=d_u, row_index=d_rows,
                                 temperatures=temps, out_draft_tokens=d_tok,
                                 want_draft_probs=False, out_row_desc=m_desc)
            sv.spec_verify_mixed_lq(z, z_rows, m_desc, d_tok, u, temps, drafter_rows=d_rows,
                                    out_tokens=out_t, out_num_accepted=acc_t, workspace=ws)
            sv.spec_verify_sample_early_exit(z, q, d, u, vi.temperature, out_tokens=out_t,
                                             out_num_accepted=acc_t, workspace=ws)
            sv.spec_verify_greedy_early_exit(z, d, out_tokens=out_t, out_num_accepted=acc_t,
                                             workspace=ws)
            sv.spec_accept_metrics(acc_t, K, mtr)
        torch.cuda.synchronize()
        # the build as two kernels (metadata, then the hidden copy) on the
        # same verify outputs, and both builds at the smaller build workload
        scall, _ = split_build(torch, out_t, acc_t, d, L, bt, bi.spec.block_size, hid, hs,
                               bi.mask_token_id)
        for i in range(args.profile_steps):
            build(); scall()
        b3 = synth.make_build_inputs(synth.build_config(3))
        o3, a3, d3 = up(b3.out_tokens), up(b3.num_accepted), up(b3.draft_tokens)
        L3, bt3, h3, hs3 = (up(b3.start_pos), up(b3.block_table), up(b3.target_hidden),
                            up(b3.h_shared))
        scall3, _ = split_build(torch, o3, a3, d3, L3, bt3, b3.spec.block_size, h3, hs3,
                                b3.mask_token_id)
        for i in range(args.profile_steps):
            sv.peagle_build_draft_batch(o3, a3, d3, L3, bt3, b3.spec.block_size, h3, hs3,
                                        b3.mask_token_id)
            scall3()
        torch.cuda.synchronize()
        # the drafter's bytes without its arithmetic (comparison kernels)
        draft_ceiling(torch, z_rows, d_rows, d_q, 1)
        torch.cuda.synchronize()
        ts = synth.TREE_CONFIGS["tree-large"]
        ti = synth.make_tree_inputs(ts, workers=1)
        tz, tq, tp, tt, tu = (up(ti.logits), up(ti.draft_probs), up(ti.parents), up(ti.tokens),
                              up(ti.uniforms))
        for i in range(args.profile_steps):
            for T in (0.0, ts.temperature):
                sv.spec_verify_tree(tz, tp, tt, T, draft_probs=tq, uniforms=tu)
                sv.spec_verify_tree_early_exit(tz, tp, tt, T, draft_probs=tq, uniforms=tu)
            ttemps = up(synth.make_temperatures(ts.B, 62))
            sv.spec_verify_tree_mixed(tz, tp, tt, ttemps, tq, tu)
        # the same trees with q from drafter logits: node (b, n) drafted from
        # the target row of node n of tree b+1 (distinct rows, so that some
        # children are rejected and the walk makes residual passes)
        nt_ = ts.B * (ts.N + 1)
        tzr = tz.view(nt_, ts.V)
        trows = ((torch.arange(nt_, dtype=torch.int32, device=dev) + ts.N + 1) % nt_).view(
            ts.B, ts.N + 1).contiguous()
        tud = up(np.random.default_rng(9).random((nt_, 1), dtype=np.float32))
        _, _, tdesc = sv.spec_draft_sample(tzr, 1, ts.temperature, uniforms=tud,
                                           row_index=trows.view(nt_, 1), want_draft_probs=False,
                                           want_row_desc=True)
        for i in range(args.profile_steps):
            sv.spec_verify_tree_lq(tz, tzr, tdesc.view(ts.B, ts.N + 1, 4), tp, tt, tu,
                                   ts.temperature, drafter_rows=trows)
        torch.cuda.synchronize()
        # the read-ceiling kernel over the logit buffer, non-temporal and cached
        rd = _stream_read_fn()
        for nt in (1, 0):
            if rd(z.data_ptr(), z.numel() * z.element_size(), nt,
                  torch.cuda.current_stream().cuda_stream):
                raise RuntimeError("svc_stream_read failed")
        torch.cuda.synchronize()
        # calibration for HBM byte counters: one plain copy of 1 GiB
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        if args.hash_out:
            os.makedirs(os.path.dirname(os.path.abspath(args.hash_out)), exist_ok=True)
            with open(args.hash_out, "w") as f:
                f.write(kernel_source_hash() + " fused\n")
        print(f"profiled {args.profile_steps} steps of every kernel family, the comparison "
              "kernels and a 1 GiB copy",
              flush=True)
        return

    def timed(sample):
        """Wall time per step with the dominant kernel traced (two events) in
        every TRACE_EVERY-th step, then every other kernel of the step timed
        the same way in a loop of its own.  The events cost ~5 us per traced
        step (measured: 0.529 against 0.524 ms per step with and without them
        on every step), so the timed loop traces a sample of its launches;
        the warmup traces every step, so that the events' first use falls
        outside the timed region."""
        dom = {"mixed": "verify_mixed_rows", True: "verify_sample_rows",
               False: "verify_greedy_rows"}[sample]
        sv.trace_begin(max(1, args.warmup), [dom])
        for _ in range(args.warmup):
            step(sample); build()
        torch.cuda.synchronize()
        sv.trace_read()
        sv.trace_end()
        sv.trace_begin((args.steps + TRACE_EVERY - 1) // TRACE_EVERY, [dom])
        torch.cuda.synchronize()
        with quiet_host():
            t0 = time.perf_counter()
            for i in range(args.steps):
                sv.trace_enable(i % TRACE_EVERY == 0)
                step(sample)
                build()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        per = {dom: [ms for _, ms in sv.trace_read()]}
        sv.trace_end()
        # per-step GPU times: one event at every step boundary on the stream
        # the library enqueues on
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        with quiet_host():
            for i in range(args.steps):
                evs[i].record()
                step(sample)
                build()
            evs[-1].record()
            torch.cuda.synchronize()
        step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
        # the step's other kernels (named from one traced step), each timed in
        # a loop of its own with only that kernel traced: two events per step,
        # so no event sits between two other kernels of the step
        sv.trace_begin(16)
        step(sample)
        build()
        torch.cuda.synchronize()
        names = [name for name, _ in sv.trace_read()]
        sv.trace_end()
        for name in names:
            if name == dom:
                continue
            sv.trace_begin(args.steps, [name])
            for _ in range(args.steps):
                step(sample)
                build()
            torch.cuda.synchronize()
            per[name] = [ms for _, ms in sv.trace_read()]
            sv.trace_end()
        acc = acc_t.cpu().numpy()
        pct = {"step_ms": percentiles(np, step_ms), dom + "_ms": percentiles(np, per[dom])}
        return wall / args.steps, {k: float(np.mean(v)) for k, v in per.items()}, acc, pct

    sec_sample, kms, acc, pct_sample = timed(True)
    vb_rows, vb_draw = verify_bytes(B, K, V, 2, acc, sample=True)
    bb = build_bytes(B, K, H, 2)
    rows = B * (K + 1)

    def kinfo(name, nbytes, note=None):
        ms = kms[name]
        d = {"avg_ms": ms, "algorithmic_bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
             "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if note:
            d["note"] = note
        return d

    res = {
        "metric": "verified logit rows/sec and achieved HBM GB/s (% of MI355X peak), 1 GPU",
        "value": rows / sec_sample,
        "unit": "verified logit rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": sec_sample * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fused high-concurrency step: sampled verify B=1024 K=7 "
                               "V=151936 bf16 logits T=0.7 + P-EAGLE build H=2048 bf16",
                   "B": B, "K": K, "V": V, "H": H, "logits": "bf16", "draft_probs": "f32",
                   "temperature": vi.temperature, "mode": "sample"},
        "step_hbm_gbs": (vb_rows + vb_draw + bb) / sec_sample / 1e9,
        "step_hbm_frac": (vb_rows + vb_draw + bb) / sec_sample / 1e9 / HBM_PEAK_GBS,
        "step_bytes": vb_rows + vb_draw + bb,
        "kernels": {
            "verify_sample_rows": kinfo("verify_sample_rows", vb_rows),
            "verify_sample_draw": kinfo("verify_sample_draw", vb_draw,
                                        "the accept scan, the residual tile masses, and "
                                        "(one workgroup per sequence) the draw of the new "
                                        "token; algorithmic bytes count the scan's reads and "
                                        "writes once and the drafter rows a_b; the kernel "
                                        "also re-reads logit row a"),
            "peagle_build": kinfo("peagle_build", bb),
        },
        "percentiles": pct_sample,
        "acceptance": {"mean_accepted": float(acc.mean()),
                       "rate": float(acc.sum() / np.minimum(acc + 1, K).sum())},
    }
    # the fused build against the same build as two kernels, on the last
    # sampled step's verify outputs
    res["build_vs_two_kernels"] = build_compare(
        torch, build, bouts, *split_build(torch, out_t, acc_t, d, L, bt, bi.spec.block_size, hid,
                                          hs, bi.mask_token_id))
    if "verify_sample_locate" in kms:
        # a separate locate kernel runs only when several draw workgroups
        # share a sequence (smaller batches)
        res["kernels"]["verify_sample_locate"] = kinfo("verify_sample_locate", B * 4)
    rk = res["kernels"]["verify_sample_rows"]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == kernel_source_hash():
            traffic = tr.get("hbm_bytes_per_launch")
    ceil = read_ceiling(torch, z, 20)
    res["roofline"] = {"bound": "hbm", "achieved": rk["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": rk["frac"], "traffic": traffic, "kernel": "verify_sample_rows",
                       "algorithmic_bytes": vb_rows, "avg_ms": rk["avg_ms"],
                       "read_ceiling_gbs": ceil["nontemporal_gbs"],
                       "frac_of_read_ceiling": rk["gbs"] / ceil["nontemporal_gbs"],
                       "traced_launches": (args.steps + TRACE_EVERY - 1) // TRACE_EVERY,
                       "traced_every": TRACE_EVERY}
    res["read_ceiling"] = ceil
    log("sampled step timed")
    if not args.no_greedy:
        sec_g, kmsg, accg, pct_g = timed(False)
        vg_rows, vg_scan = verify_bytes(B, K, V, 2, accg, sample=False)
        g_ms = kmsg["verify_greedy_rows"]
        res["greedy_step"] = {"value": rows / sec_g, "unit": "verified logit rows/s",
                              "ms_per_step": sec_g * 1e3,
                              "verify_greedy_rows": {"avg_ms": g_ms, "algorithmic_bytes": vg_rows,
                                                     "gbs": vg_rows / (g_ms * 1e-3) / 1e9,
                                                     "frac": vg_rows / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                              "verify_greedy_accept_ms": kmsg["verify_greedy_accept"],
                              "percentiles": pct_g,
                              "peagle_build_ms": kmsg["peagle_build"],
                              "step_hbm_gbs": (vg_rows + vg_scan + bb) / sec_g / 1e9,
                              "step_hbm_frac": (vg_rows + vg_scan + bb) / sec_g / 1e9 / HBM_PEAK_GBS}
    if not args.no_greedy:
        sec_m, kmsm, accm, _ = timed("mixed")
        sampled = temps_np > 0
        vm_rows, _ = verify_bytes(B, K, V, 2, accm, sample=True)
        # scan bytes: greedy sequences as in greedy mode, sampled ones as in sampling
        ns = int(sampled.sum())
        vm_draw = (B * K * 4 + B * (K + 1) * 4 + B * 4 + B * 4
                   + ns * (K * 4 * 3 + (K + 1) * 4)
                   + int(((accm < K) & sampled).sum()) * V * 4)
        res["mixed_step"] = {
            "value": rows / sec_m, "unit": "verified logit rows/s", "ms_per_step": sec_m * 1e3,
            "workload": "the fused batch with per-sequence temperatures "
                        f"({int((~sampled).sum())} greedy, {int(sampled.sum())} sampled), + build",
            "kernels_ms": {k: v for k, v in kmsm.items()},
            "step_hbm_gbs": (vm_rows + vm_draw + bb) / sec_m / 1e9,
            "step_hbm_frac": (vm_rows + vm_draw + bb) / sec_m / 1e9 / HBM_PEAK_GBS}
        log("mixed step timed")
    if not args.no_early_exit:
        res["early_exit"] = early_exit_bench(sv, torch, np, args, B, K, V, vi, bi, z, q, d, u,
                                             temps, L, bt, hid, hs, ws, bouts)
        log("early-exit verify timed")
    if not args.no_graph:
        res["graph_step"] = graph_bench(sv, torch, np, args, B, K, V, vi, bi, z, q, d, u, L, bt,
                                        hid, hs, out_t, acc_t, pd_t, ws, bouts)
        log("graph step timed")
    if not args.no_draft:
        def timed_draft(with_q):
            for _ in range(args.warmup):
                draft(with_q)
            torch.cuda.synchronize()
            sv.trace_begin(args.steps, ["draft_sample"])
            for _ in range(args.steps):
                draft(with_q)
            torch.cuda.synchronize()
            ms = float(np.mean([m for _, m in sv.trace_read()]))
            sv.trace_end()
            nbytes = B * K * (V * 2 + (V * 4 if with_q else 0) + 12)
            return {"avg_ms": ms, "rows_per_s": B * K / (ms * 1e-3), "algorithmic_bytes": nbytes,
                    "gbs": nbytes / (ms * 1e-3) / 1e9,
                    "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        res["draft_sample"] = {
            "workload": f"drafter-output sampling B={B} K={K} V={V} bf16 T={vi.temperature}: "
                        "K draft tokens per sequence and their fp32 distributions",
            "with_probs": timed_draft(True),
            "tokens_only": timed_draft(False),
            "copy_ceiling": draft_ceiling(torch, z_rows, d_rows, d_q, 10)}
        log("drafter sampling timed")
    if not args.no_round:
        res["decode_round"] = round_bench(sv, torch, np, args, B, K, V, vi, bi, z, d, u, L, bt,
                                          hid, hs, out_t, acc_t, pd_t, ws, bouts, temps)
        log("decode round timed")
    if not args.no_tree:
        res["tree_verify"] = tree_bench(sv, torch, np, synth, args)
        log("tree verify timed")
    if not args.no_small:
        res["small_workloads"] = small_workloads_bench(sv, torch, np, synth, args)
        log("smaller workloads timed")
        res["fp32_logits"] = fp32_bench(sv, torch, np, args, vi, z, q, d, u, ws)
        log("fp32 logits timed")
    if args.cpu_budget > 0:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(vi, bi, args.cpu_budget)
        res["cpu_baseline_all_cores"] = cpu_all
        # the same algorithmic bytes per sequence as the GPU step
        per_seq = res["step_bytes"] / B
        for key in ("cpu_baseline", "cpu_baseline_all_cores"):
            if res.get(key):
                res[key]["gbs_algorithmic"] = res[key]["value"] / (K + 1) * per_seq / 1e9
    res["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
