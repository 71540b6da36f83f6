"""CPU: the rocprofv3 summary arithmetic (per-launch sums over a plan's
kernels, counter means per dispatch, HBM bytes scaled by the copy kernel's
reading) on synthetic CSV files in the layout rocprofv3 writes."""
import csv
import os
import types

from tiled_software_pipelined_amd import profiling


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _passes(out, rcs, start=0.0):
    """passes.json as collect() writes it: every pass started at `start`."""
    import json
    os.makedirs(str(out), exist_ok=True)
    with open(str(out / profiling.PASSES_FILE), "w") as f:
        json.dump({name: {"rc": rc, "start": start} for name, rc in rcs.items()}, f)


ALL_OK = {"trace": 0, "pmc0": 0, "pmc1": 0, "pmc2": 0, "pmc3": 0, "pmc4": 0}


def test_split_plan_sums_its_kernels(tmp_path):
    out = tmp_path / "prof"
    _passes(out, ALL_OK)
    main = "void tg::gemm_kernel<tg::MfmaGemm<...>, 2>(tg::GemmArgs)"
    thin = "void tg::gemm_kernel<tg::ThinGemm<1, 1>, 2>(tg::GemmArgs)"
    _write(str(out / "trace" / "x" / "trace_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [[main, 25, 25 * 200000, 200000, 90, 190000, 230000, 1], [thin, 25, 25 * 15000, 15000, 7, 14000, 17000, 1],
            ["elementwise_copy", 3, 300, 100, 3, 90, 110, 1]])
    # FETCH_SIZE (group 2) and WRITE_SIZE (group 3): two dispatches of each
    # GEMM kernel, one of the copy
    rows = []
    for name, vals in ((main, (1000.0, 1200.0)), (thin, (100.0, 100.0))):
        for v in vals:
            rows.append([name, "FETCH_SIZE", v])
    rows.append(["elementwise_copy_kernel", "FETCH_SIZE", 2.0 ** 28 / 2048.0])  # 2 KiB per unit
    _write(str(out / "pmc2" / "x" / "pmc_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
           rows)
    rows = [[main, "WRITE_SIZE", 500.0], [main, "WRITE_SIZE", 500.0], [thin, "WRITE_SIZE", 4.0],
            ["elementwise_copy_kernel", "WRITE_SIZE", 2.0 ** 28 / 1024.0]]  # 1 KiB per unit
    _write(str(out / "pmc3" / "x" / "pmc_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
           rows)
    args = types.SimpleNamespace(out=str(out), workload="bf16_4096", variant="", steps=20, warmup=5)
    res = profiling.summarize(args, {})
    assert [k["name"] for k in res["kernels"]] == [main, thin]
    assert res["avg_ns"] == 215000 and res["min_ns"] == 204000 and res["calls"] == 25
    # counters: each kernel's mean per dispatch, added over the plan's kernels
    assert res["counters"]["FETCH_SIZE"] == 1100.0 + 100.0
    assert res["counters"]["WRITE_SIZE"] == 500.0 + 4.0
    # bytes per counter unit = the calibration copy's size / its reading
    calib = profiling.CALIB_MIB << 20
    fetch_scale = calib / res["copy"]["FETCH_SIZE"]
    write_scale = calib / res["copy"]["WRITE_SIZE"]
    assert fetch_scale == calib / (2.0 ** 28 / 2048.0)
    assert write_scale == calib / (2.0 ** 28 / 1024.0)


def test_kernel_resources_from_trace():
    rows = [{"Kernel_Name": "void tg::gemm_kernel<tg::MfmaGemm<...>, 2>(tg::GemmArgs)", "LDS_Block_Size": "131072",
             "Scratch_Size": "0", "Workgroup_Size_X": "512", "Workgroup_Size_Y": "1", "Workgroup_Size_Z": "1"},
            {"Kernel_Name": "tg::pack_rows(char const*, char*, long, long, long, long)", "LDS_Block_Size": "0",
             "Scratch_Size": "0", "Workgroup_Size_X": "256", "Workgroup_Size_Y": "1", "Workgroup_Size_Z": "1"},
            {"Kernel_Name": "elementwise_copy_kernel", "LDS_Block_Size": "0", "Scratch_Size": "0",
             "Workgroup_Size_X": "128", "Workgroup_Size_Y": "1", "Workgroup_Size_Z": "1"}]
    res = profiling.kernel_resources(rows)
    assert set(res) == {rows[0]["Kernel_Name"], rows[1]["Kernel_Name"]}
    main = res[rows[0]["Kernel_Name"]]
    assert main["lds_bytes"] == 131072 and main["wg_per_cu_by_lds"] == 1 and main["threads"] == 512
    assert res[rows[1]["Kernel_Name"]]["wg_per_cu_by_lds"] is None


def test_runtime_occupancy_line(tmp_path):
    # the collected workgroups-per-CU figure is used only for the kernel the
    # plan runs, with threads and LDS from the trace
    import json

    out = tmp_path / "prof"
    os.makedirs(out)
    args = types.SimpleNamespace(out=str(out), workload="bf16_4096", variant="", steps=20, warmup=5)
    from tiled_software_pipelined_amd import inputs
    w = inputs.workloads()["bf16_4096"]
    kname = profiling._plan_name(args, w)
    main = "void tg::gemm_kernel<tg::MfmaGemm<...>, 2>(tg::GemmArgs)"
    res = {"kernel": main, "resources": {main: {"threads": 512, "lds_bytes": 131072, "scratch": 0,
                                               "wg_per_cu_by_lds": 1}}}
    assert profiling._runtime_occupancy(args, w, res) is None  # nothing recorded
    with open(out / profiling.OCC_FILE, "w") as f:
        json.dump({"kernel": kname, "workgroups_per_cu": 1}, f)
    assert profiling._runtime_occupancy(args, w, res) == (512, 131072, 1, 2.0)
    with open(out / profiling.OCC_FILE, "w") as f:
        json.dump({"kernel": "some_other_kernel", "workgroups_per_cu": 3}, f)
    assert profiling._runtime_occupancy(args, w, res) is None


def _one_fetch_pass(out):
    main = "void tg::gemm_kernel<tg::MfmaGemm<...>, 2>(tg::GemmArgs)"
    _write(str(out / "pmc2" / "x" / "pmc_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
           [[main, "FETCH_SIZE", 1000.0], ["elementwise_copy_kernel", "FETCH_SIZE", 512.0]])
    return types.SimpleNamespace(out=str(out), workload="bf16_4096", variant="", steps=20, warmup=5)


def test_pass_without_record_is_not_used(tmp_path):
    out = tmp_path / "prof"
    args = _one_fetch_pass(out)
    res = profiling.summarize(args, {})
    assert "FETCH_SIZE" not in res["counters"]
    assert res["passes"]["pmc2"]["status"].startswith("no record")


def test_stale_csv_is_not_used(tmp_path):
    import time
    out = tmp_path / "prof"
    args = _one_fetch_pass(out)
    _passes(out, {"pmc2": 0}, start=time.time() + 3600)  # the file predates the pass
    res = profiling.summarize(args, {})
    assert "FETCH_SIZE" not in res["counters"] and res["passes"]["pmc2"]["status"].startswith("stale")


def test_killed_pass_without_csv_is_reported(tmp_path):
    out = tmp_path / "prof"
    _passes(out, {"trace": 0, "pmc2": 137})
    args = types.SimpleNamespace(out=str(out), workload="bf16_4096", variant="", steps=20, warmup=5)
    res = profiling.summarize(args, {})
    assert res["passes"]["pmc2"] == {"rc": 137, "csv": None, "status": "no CSV written"}
    assert res["counters"] == {}


def test_fresh_csv_with_nonzero_exit_is_used_and_flagged(tmp_path):
    out = tmp_path / "prof"
    args = _one_fetch_pass(out)
    _passes(out, {"pmc2": 139}, start=0.0)
    res = profiling.summarize(args, {})
    assert res["counters"]["FETCH_SIZE"] == 1000.0
    assert res["passes"]["pmc2"]["status"] == "ok (CSV complete; exit status 139)"
