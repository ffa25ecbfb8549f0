"""Host logic of bench.py: the algorithmic byte count behind the roofline and
the conversion of rocprofv3 counter CSVs into HBM bytes per launch."""
from __future__ import annotations

import csv
import os

import bench


def test_algorithmic_bytes_headline():
    # 8 x 2048 tokens, 16 heads, fp32 state read and written:
    # 16384 * 16 * (4 * 256 + 2 + 256) + 8 * 16 * 2 * 65536
    assert bench.algorithmic_bytes(16384, 16, 8, 4, True) == 352_845_824
    # no initial state: the state is only written; bf16 halves it
    assert bench.algorithmic_bytes(16384, 16, 8, 4, False) == 16384 * 16 * 1282 + 8 * 16 * 65536
    assert bench.algorithmic_bytes(256, 2, 1, 2, True) == 256 * 2 * 1282 + 2 * 2 * 32768


def _write_counters(path, kernel, values_per_dispatch):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for d, vals in enumerate(values_per_dispatch):
            for v in vals:  # several rows (e.g. per XCD) summed per dispatch
                w.writerow(dict(Dispatch_Id=d, Kernel_Name=kernel, Counter_Name="X",
                                Counter_Value=v))


def test_traffic_from_counters(tmp_path):
    pmc = str(tmp_path)
    k = "void kda::(anonymous namespace)::pipe_kernel<64>(kda::Params)"
    _write_counters(os.path.join(pmc, "fetch", "run_counter_collection.csv"), k,
                    [[600.0, 400.0], [500.0, 500.0]])          # 1000 KiB per dispatch
    _write_counters(os.path.join(pmc, "write", "run_counter_collection.csv"), k,
                    [[250.0, 250.0]])                           # 500 KiB per dispatch
    # the calibration copy of 256 MiB reads as half its bytes on FETCH_SIZE and
    # all of them on WRITE_SIZE: scales x2 and x1
    _write_counters(os.path.join(pmc, "cal_fetch", "run_counter_collection.csv"),
                    "__amd_rocclr_copyBuffer", [[128 * 1024.0]])
    _write_counters(os.path.join(pmc, "cal_write", "run_counter_collection.csv"),
                    "__amd_rocclr_copyBuffer", [[256 * 1024.0]])
    t = bench.traffic_from_pmc(pmc, "w", "cmd", "pipe_kernel")
    assert t["fetch_kib_per_dispatch"] == 1000.0 and t["write_kib_per_dispatch"] == 500.0
    assert t["dispatches"] == [2, 1]
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["bytes_per_launch"] == (1000.0 * 2.0 + 500.0) * 1024.0
    assert t["kernel_source_sha256"] == bench.kernel_source_hash()


def test_dominant_kernel_follows_the_library_choice():
    import bench
    assert bench.dominant_kernel(True, -5.0) == "decode_kernel"
    assert bench.dominant_kernel(False, -5.0) == "pipe_kernel"
    assert bench.dominant_kernel(False, -1.0) == "pipe_kernel"
    assert bench.dominant_kernel(False, -5.25) == "fwd32_kernel"
    seg = bench.dominant_kernel(False, -5.0, 2048, 64)
    assert seg.split("+") == ["seg_plan_kernel", "pipe_kernel<64, true>", "seg_combine_kernel",
                              "pipe_kernel<64, false>"]
    assert bench.traffic_file("w", seg).endswith(
        "traffic__seg_plan_kernel+pipe_kernel64_true+seg_combine_kernel+pipe_kernel64_false__w.json")


def test_bench_labels_the_segmented_workloads():
    """configs 2 and 3 (one or two long sequences, few heads) take the
    segment-parallel schedule; config 1 does not; --segments off turns it off."""
    import argparse
    import bench
    a = argparse.Namespace(proj=0, decode_batch=0, config=2, lower_bound=None, segments="auto",
                           vsplit=0, checkpoint_interval=0, uniform=None)
    assert bench.workload_name(a)[1].startswith("seg_plan_kernel+")
    a.config = 3
    assert bench.workload_name(a)[1].startswith("seg_plan_kernel+")
    a.config = 1
    assert bench.workload_name(a)[1] == "pipe_kernel"
    a.config, a.segments = 2, "off"
    assert bench.workload_name(a)[1] == "pipe_kernel"
    a.segments = "auto"
    bench.apply_hooks(a)


def test_bench_labels_the_two_workgroup_workloads():
    """A uniform workload in the two-workgroup form's range is labelled with
    its kernel; the 8 x 2048, 16-head configuration is not in that range."""
    import argparse
    import bench
    a = argparse.Namespace(proj=0, decode_batch=0, config=1, lower_bound=None, segments="auto",
                           vsplit=0, checkpoint_interval=0, uniform="32,512,4")
    wl, kern, sel = bench.workload_name(a)
    assert (wl, kern, sel) == ("uniform_32x512_h4", "duo_kernel", "--uniform 32,512,4")
    a.uniform = None
    assert bench.workload_name(a)[1] == "pipe_kernel"
    a.uniform, a.vsplit = "32,512,4", 2
    assert bench.workload_name(a)[1] == "pipe_kernel"
    a.uniform, a.vsplit, a.kernel = None, 0, 6     # forced: the headline shape in two workgroups
    assert bench.workload_name(a) == ("varlen_8x2048_h16_kernel6", "duo_kernel", "--config 1 --kernel 6")
    bench.apply_hooks(argparse.Namespace(segments="auto", vsplit=0, kernel=0))
