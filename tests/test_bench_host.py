"""Host-side logic of bench.py (no GPU): the traffic record's source digest
and the effective-clock summary of a counter run."""
import csv
import json
import os

import bench


def test_code_only_drops_comments_and_blank_space():
    src = "int a = 1;  // the count\n/* block\n   comment */\nint  b =\t2; // end"
    assert bench._code_only(src) == "int a = 1; int b = 2;"
    # a comment edit leaves the code digest unchanged, a code edit does not
    assert bench._code_only(src.replace("the count", "a count")) == bench._code_only(src)
    assert bench._code_only(src.replace("2;", "3;")) != bench._code_only(src)


def test_source_digest_is_stable():
    assert bench.source_digest() == bench.source_digest()
    assert len(bench.source_digest()) == 16


def _write_run(d, rows, n_xcc=8):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_agent_info.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Node_Id", "Agent_Type", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Node_Id": 0, "Agent_Type": "CPU", "Num_Xcc": 0})
        w.writerow({"Node_Id": 1, "Agent_Type": "GPU", "Num_Xcc": n_xcc})
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value",
                                           "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_clock_summary(tmp_path):
    run = str(tmp_path / "run")
    ms = 1_000_000
    rows = [
        # 5 ms at 1.6 GHz on each of 8 XCDs
        {"Kernel_Name": "moe::k_gate_up_bf16(moe::GroupedArgs)", "Counter_Name": "GRBM_GUI_ACTIVE",
         "Counter_Value": 1.6 * 5 * ms * 8, "Start_Timestamp": 0, "End_Timestamp": 5 * ms},
        {"Kernel_Name": "moe::k_gate_up_bf16(moe::GroupedArgs)", "Counter_Name": "GRBM_GUI_ACTIVE",
         "Counter_Value": 1.8 * 5 * ms * 8, "Start_Timestamp": 0, "End_Timestamp": 5 * ms},
        {"Kernel_Name": "moe::k_gate_up_bf16(moe::GroupedArgs)", "Counter_Name": "GRBM_GUI_ACTIVE",
         "Counter_Value": 1.7 * 5 * ms * 8, "Start_Timestamp": 0, "End_Timestamp": 5 * ms},
        # too short to count: the counter window inflates it
        {"Kernel_Name": "moe::k_fill_i32(int*, int, int)", "Counter_Name": "GRBM_GUI_ACTIVE",
         "Counter_Value": 1e9, "Start_Timestamp": 0, "End_Timestamp": 2000},
        # another counter is ignored
        {"Kernel_Name": "moe::k_down_bf16(moe::GroupedArgs)", "Counter_Name": "SQ_WAVES",
         "Counter_Value": 5, "Start_Timestamp": 0, "End_Timestamp": 3 * ms},
    ]
    _write_run(run, rows)
    out = str(tmp_path / "clock.json")
    bench.clock_summary(run, "v3_prefill", path=out)
    rec = json.load(open(out))
    assert rec["xcds"] == 8
    k = rec["kernels"]
    assert set(k) == {"moe::k_gate_up_bf16"}
    assert k["moe::k_gate_up_bf16"]["dispatches"] == 3
    assert abs(k["moe::k_gate_up_bf16"]["ghz_median"] - 1.7) < 1e-9
    assert abs(k["moe::k_gate_up_bf16"]["ghz_min"] - 1.6) < 1e-9
    assert abs(k["moe::k_gate_up_bf16"]["ms_median"] - 5.0) < 1e-9
