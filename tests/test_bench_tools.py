"""CPU checks of bench.py's accounting: the algorithmic work of each configuration, and the
profile summariser's byte-counter arithmetic on a small synthetic set of rocprofv3 csv files."""
import csv
import os

import pytest

import bench
import workloads as wl

# algorithmic flops and bytes of the configurations, computed independently from their
# definitions (flops: 2 (576 + 512) H per visible (row, key) pair; bytes: key rows and
# indices, q, fp32 out, mask tails, indptrs)
EXPECTED = {
    "tiny": (4.63e6, 296_536),
    "short": (12.71e9, 9_907_656),
    "long": (51.26e9, 29_975_656),
    "segmented": (212.8e9, 122_009_788),
    "stress": (2336.5e9, 330_458_172),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_work(name):
    w = wl.make(name)
    by, fl = bench.algorithmic_work(w)
    fl_ref, by_ref = EXPECTED[name]
    assert abs(fl - fl_ref) <= 0.0005 * fl_ref
    assert by == by_ref


def test_long_flops_from_visible_pairs():
    """The long config's flops counted pair by pair from its mask: P keys for every row plus
    each tree token's visible tree keys."""
    w = wl.make("long")
    t, p = int(w.tree_lens[0]), int(w.prefix_lens[0])
    m = w.custom_mask.reshape(t, p + t)
    pairs = w.num_heads * (t * p + int((m[:, p:] != 0).sum()))
    assert bench.algorithmic_work(w)[1] == 2 * (576 + 512) * pairs


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_summarize_profile_scales_the_byte_counters(tmp_path):
    out = tmp_path / "prof"
    k = "void va::(anonymous namespace)::mfma_partial_kernel<false>(va::RunArgs, va::Workspace, int)"
    cal = "void at::native::elementwise_kernel<MulFunctor>(...)"
    tr_head = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
               "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
               "Workgroup_Size_X", "Grid_Size_X"]
    _write_csv(str(out / "trace" / "run_kernel_trace.csv"), tr_head, [
        ["KERNEL_DISPATCH", 1, k, 1000, 71000, 161792, 0, 256, 0, 112, 256, 65536],
        ["KERNEL_DISPATCH", 2, k, 100000, 172000, 161792, 0, 256, 0, 112, 256, 65536],
    ])
    _write_csv(str(out / "trace" / "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                "StdDev"], [[k, 2, 142000, 71000.0, 70.0, 70000, 72000, 1000.0]])
    cc_head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # two instances per dispatch summed; the calibration reads 131072 KiB (factor 2) and
    # writes 262144 KiB (factor 1)
    _write_csv(str(out / "fetch" / "run_counter_collection.csv"), cc_head, [
        [1, k, "FETCH_SIZE", 9000.0], [1, k, "FETCH_SIZE", 9000.0],
        [2, k, "FETCH_SIZE", 9000.0], [2, k, "FETCH_SIZE", 9000.0],
        [3, cal, "FETCH_SIZE", 131072.0],
    ])
    _write_csv(str(out / "write" / "run_counter_collection.csv"), cc_head, [
        [1, k, "WRITE_SIZE", 30000.0], [2, k, "WRITE_SIZE", 34000.0],
        [3, cal, "WRITE_SIZE", 262144.0],
    ])
    (out / "trace.json").write_text('{"partial_kernel_us": 71.0, "combine_kernel_us": 11.0, '
                                    '"value": 88.0}\n')
    dest = tmp_path / "summaries"
    dest.mkdir()
    paths = bench.summarize_profile(str(out), "long", dest=str(dest))
    assert [os.path.basename(p) for p in paths] == ["mfma_partial_kernel_long.txt"]
    text = open(paths[0]).read()
    # (18000 KiB x 2 + 32000 KiB x 1) x 1024 bytes
    assert f"traffic per dispatch: {(18000 * 2 + 32000) * 1024} bytes" in text
    assert "average 71.000 us, median 71.000 us" in text
    assert "calls 2, average 71.000 us" in text
    assert "bench.py --workload long --summarize-profile <out>" in text


def test_timed_dispatches_slice_after_the_settle_and_warmup_steps():
    # 1 checked call, 3 settle steps, 2 warm-up steps, then 4 timed steps, then replays
    d = [50.0] + [80.0] * 3 + [70.0] * 2 + [60.0, 62.0, 64.0, 66.0] + [90.0] * 5
    line = bench._timed_dispatches(d, {"settle_steps": 3, "warmup": 2, "steps": 4},
                                   "mfma_partial_ws_kernel")
    assert line == ["  the 4 timed steps (dispatches 6..9): average 63.000 us, min 60.000 us, "
                    "max 66.000 us"]
    # the tree kernels are not launched once per step; too few dispatches give nothing either
    assert bench._timed_dispatches(d, {"settle_steps": 3, "warmup": 2, "steps": 4},
                                   "build_mask_kernel") == []
    assert bench._timed_dispatches(d[:8], {"settle_steps": 3, "warmup": 2, "steps": 4},
                                   "combine_kernel") == []
