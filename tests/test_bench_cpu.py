"""Host logic of bench.py, without a GPU.

* More than one GPU is refused with a message, before anything is imported
  that touches a device.
* The algorithmic byte counts of the fused step are the sizes of the arrays
  the method reads and writes once (8192 logit rows of 151936 bf16 values;
  the build's hidden rows), as stated for the workload.
* Counter ingestion: per-kernel bytes are the counter's KiB scaled by what
  the same counter reads for the 1 GiB calibration copy, kernels that serve
  several workloads are kept apart by grid size, the dominant kernel is the
  sampled row kernel of the largest grid, and counters recorded on other
  kernel sources are refused.
* The comparison library (read ceiling, the drafter's bytes without its
  arithmetic, the two-kernel build) loads without a GPU and refuses invalid
  arguments before launching anything.
"""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]
ROWS_S = "void sv::verify_rows<unsigned short, 1, true>(sv::RowsArgs)"
COPY = "__amd_rocclr_copyBuffer"


def test_read_ceiling_library_exports_and_rejects_bad_arguments():
    """The streaming-read kernel's library loads without a GPU; invalid
    arguments are refused before anything is launched."""
    import ctypes
    if not os.path.exists(bench.CEILING_LIB):
        pytest.skip("libsvceiling.so is not built")
    fn = ctypes.CDLL(bench.CEILING_LIB).svc_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    assert fn(None, 1024, 1, None) == 1                   # no buffer
    assert fn(16, 0, 1, None) == 1                        # no bytes
    assert fn(16, 1000, 0, None) == 1                     # not a multiple of 16
    assert fn(8, 1024, 0, None) == 1                      # not 16-byte aligned
    lib = ctypes.CDLL(bench.CEILING_LIB)
    vp, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    cvt = lib.svc_rows_to_f32
    cvt.argtypes = [vp, vp, i64, vp, i64, i, i, vp]
    assert cvt(None, 16, 8, 16, 4, 64, 1, None) == 1       # no source rows
    assert cvt(16, 16, 8, 16, 4, 60, 1, None) == 1         # V not a multiple of 8
    assert cvt(16, 16, 8, 16, 0, 64, 1, None) == 1         # no output rows
    assert cvt(8, 16, 8, 16, 4, 64, 1, None) == 1          # source not 16-byte aligned
    wr = lib.svc_write_rows
    wr.argtypes = [vp, i64, i, i, vp]
    assert wr(None, 4, 64, 1, None) == 1
    assert wr(16, 4, 62, 1, None) == 1                    # V not a multiple of 4
    assert wr(16, -1, 64, 1, None) == 1
    sb = lib.svc_build_split
    sb.argtypes = [vp] * 5 + [i, i, vp, vp, ctypes.c_int32, i, i, i] + [vp] * 7
    args = [16] * 5 + [4, 16, 16, 16, 7, 8, 7, 2048] + [16] * 6 + [None]
    for pos, bad in ((11, 0), (11, 64), (12, 12), (10, 0), (16, None), (18, None), (7, 8)):
        a = list(args)
        a[pos] = bad                                      # K, H, B, an output, alignment
        assert sb(*a) == 1, pos


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_algorithmic_bytes_of_the_fused_step():
    B, K, V, H = 1024, 7, 151936, 2048
    acc = np.full(B, 3)                       # every sequence rejects draft 3
    rows, rest = bench.verify_bytes(B, K, V, 2, acc, sample=True)
    assert rows == 8192 * 303_872 == 2_489_319_424
    # the drafter row of every rejecting sequence dominates the rest
    assert rest - B * V * 4 == B * (K * 4 + (K + 1) * 4 + 4 + K * 8 + (K + 1) * 4 + K * 4)
    rows_g, rest_g = bench.verify_bytes(B, K, V, 2, acc, sample=False)
    assert rows_g == rows and rest_g == B * (K * 4 + (K + 1) * 4 + 4)
    # a batch that accepts everything reads no drafter row
    assert bench.verify_bytes(B, K, V, 2, np.full(B, K))[1] == rest - B * V * 4
    build = bench.build_bytes(B, K, H, 2)
    hidden = (B * (K + 1) + 1 + B * 2 * K) * H * 2   # verify rows + h_shared read, 2K rows written
    assert hidden < build < hidden + 1_000_000
    assert abs(build / 1e6 - 92.7) < 0.1


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, kib) in enumerate(rows):
            w.writerow({**{k: 0 for k in FIELDS}, "Dispatch_Id": i + 1, "Grid_Size": grid,
                        "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib,
                        "Start_Timestamp": 1000, "End_Timestamp": 2000})


def _run_ingest(tmp_path, monkeypatch, hash_on_disk="abc123"):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.json"))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    for d in ("f", "w"):
        os.makedirs(tmp_path / d)
        (tmp_path / d / "source_hash.txt").write_text(hash_on_disk + "\n")
    # the copy reads 1 GiB and writes 1 GiB; FETCH_SIZE counts half of it
    _csv(tmp_path / "f" / "f_counter_collection.csv", "FETCH_SIZE",
         [(COPY, 512, 4.0), (COPY, 268435456, 524288.0),
          (ROWS_S, 524288, 1000.0), (ROWS_S, 2097152, 1_215_525.0), (ROWS_S, 2097152, 1_215_527.0),
          ("void at::native::some_torch_kernel", 64, 9.0)])
    _csv(tmp_path / "w" / "w_counter_collection.csv", "WRITE_SIZE",
         [(COPY, 512, 4.0), (COPY, 268435456, 1_048_576.0),
          (ROWS_S, 524288, 2.0), (ROWS_S, 2097152, 128.0), (ROWS_S, 2097152, 128.0)])
    bench.ingest_counters(str(tmp_path / "f" / "f_counter_collection.csv"),
                          str(tmp_path / "w" / "w_counter_collection.csv"))
    return json.load(open(tmp_path / "profiles" / "traffic.json"))


def test_counter_ingestion(tmp_path, monkeypatch, capsys):
    rec = _run_ingest(tmp_path, monkeypatch)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["source_hash"] == "abc123"
    big = f"{ROWS_S} [grid 2097152]"
    assert rec["kernel"] == big
    k = rec["kernels"][big]
    assert k["dispatches"] == 2
    assert k["fetch_bytes"] == 1_215_526.0 * 1024 * 2
    assert k["write_bytes"] == 128.0 * 1024
    assert rec["hbm_bytes_per_launch"] == k["fetch_bytes"] + k["write_bytes"]
    small = rec["kernels"][f"{ROWS_S} [grid 524288]"]
    assert small["fetch_bytes"] == 1000.0 * 1024 * 2 and small["dispatches"] == 1
    assert not any("torch" in name or "copyBuffer" in name for name in rec["kernels"])
    md = open(tmp_path / "profiles" / "hbm_counters_fused_b1024.md").read()
    assert "FETCH_SIZE x 2.0000" in md and "--pmc FETCH_SIZE" in md and "--pmc WRITE_SIZE" in md


def test_counters_from_other_sources_are_refused(tmp_path, monkeypatch):
    with pytest.raises(SystemExit) as e:
        _run_ingest(tmp_path, monkeypatch, hash_on_disk="feedbeef")
    assert "feedbeef" in str(e.value)
    assert not os.path.exists(tmp_path / "profiles" / "traffic.json")


def test_tree_walk_passes_hand_example():
    """Row passes of the sampled tree walk, counted from the path: root with
    children 1 and 2, node 1 with child 3, node 2 with child 4.  A rejected
    child costs one residual pass; a leaf at the end of the path costs one
    logit-only pass (the tile masses of the target distribution)."""
    parents = np.array([[0, 0, 1, 2]] * 4, np.int32)
    path = np.array([[-1, -1, -1, -1, -1],     # both root children rejected
                     [2, -1, -1, -1, -1],      # 1 rejected, 2 accepted, then 4 rejected
                     [1, 3, -1, -1, -1],       # 1 and 3 accepted, 3 is a leaf
                     [1, -1, -1, -1, -1]],     # 1 accepted, then 3 rejected
                    np.int32)
    acc = np.array([0, 1, 2, 1], np.int32)
    res, plain = bench.tree_walk_passes(np, parents, path, acc)
    assert res.tolist() == [2, 2, 0, 1]
    assert plain.tolist() == [0, 0, 1, 0]


def test_trace_ingestion_summarises_per_kernel_and_grid(tmp_path, monkeypatch):
    """The kernel trace summary averages each (kernel, grid size) pair over
    its dispatches, refuses a trace taken on other kernel sources, and names
    the dominant kernel's average."""
    os.makedirs(tmp_path / "profiles")
    os.makedirs(tmp_path / "t")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    path = tmp_path / "t" / "st_kernel_trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
                    "Start_Timestamp", "End_Timestamp"])
        w.writerow([ROWS_S, 524288, 1, 1, 800000, 850000])   # the same kernel, a smaller batch
        w.writerow([ROWS_S, 2097152, 1, 1, 0, 360000])       # ns
        w.writerow([ROWS_S, 2097152, 1, 1, 400000, 770000])
    (tmp_path / "t" / "source_hash.txt").write_text("other\n")
    with pytest.raises(SystemExit):
        bench.ingest_trace(str(path))
    (tmp_path / "t" / "source_hash.txt").write_text("abc123\n")
    bench.ingest_trace(str(path))
    md = (tmp_path / "profiles" / "kernel_trace_fused_b1024.md").read_text()
    assert f"| `{ROWS_S}` | 2097152 | 2 | 365.0 | 360.0 | 370.0 |" in md
    assert f"| `{ROWS_S}` | 524288 | 1 | 50.0 | 50.0 | 50.0 |" in md
    assert "grid 2097152): 365.0 µs average over 2 dispatches" in md   # the largest grid
