"""The LDS and vector-memory table that bench.py writes from a rocprofv3 counter run: its
shares and rates follow from the counters by the stated formulas (LDS busy is rocprofv3's
LdsUtil: SQ_LDS_IDX_ACTIVE over elapsed cycles x CUs, the elapsed cycles being
GRBM_GUI_ACTIVE over the 8 XCDs), checked on a synthetic counter file with known answers."""

import csv
import os

import bench

CUS = 256


def _write_counters(path, kernel, dur_ns, counters, dispatch=1):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
                                          "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in counters.items():
            w.writerow({"Dispatch_Id": dispatch, "Kernel_Name": kernel, "Start_Timestamp": 1000,
                        "End_Timestamp": 1000 + dur_ns, "Counter_Name": name, "Counter_Value": value})


def test_lds_table_shares(tmp_path):
    elapsed = 150_000  # cycles of one XCD over a 100 us dispatch: 1.5 GHz
    counters = {
        "GRBM_GUI_ACTIVE": 8 * elapsed,
        "SQ_LDS_IDX_ACTIVE": 0.25 * CUS * elapsed,            # 25% busy
        "SQ_INSTS_LDS_LOAD_BANDWIDTH": 80 * CUS * elapsed / 64,  # 80 bytes per CU per cycle
        "SQ_INSTS_LDS_STORE_BANDWIDTH": 2 * CUS * elapsed / 64,  # 2 bytes per CU per cycle
        "SQ_LDS_BANK_CONFLICT": 0.1 * 0.25 * CUS * elapsed,   # 10% of the busy cycles
        "SQ_LDS_DATA_FIFO_FULL": 0.03 * CUS * elapsed,
        "TA_BUSY_avr": 0.5 * elapsed,                         # mean over the TA instances
        "TD_TD_BUSY_sum": 0.75 * CUS * elapsed,               # summed over the CUs
        "SQ_VMEM_TA_ADDR_FIFO_FULL": 0.0,
        "SQ_BUSY_CU_CYCLES": 0.0,
    }
    _write_counters(os.path.join(tmp_path, "lds_counter_collection.csv"), "probe_kernel(int)", 100_000, counters)
    lines = bench._summarize_lds(str(tmp_path))
    rows = [ln for ln in lines if ln.startswith("| `probe_kernel")]
    assert len(rows) == 1
    cells = [c.strip() for c in rows[0].strip("|").split("|")]
    # kernel, us, clock, LDS busy, read B/clk, written B/clk, conflict, data queue full, TA, TD, TA queue full
    assert cells[1:] == ["100.0", "1.50", "25.0%", "80.0", "2.0", "10.0%", "3.0%", "50.0%", "75.0%", "0.0%"]


def test_lds_table_skips_short_dispatches(tmp_path):
    _write_counters(os.path.join(tmp_path, "lds_counter_collection.csv"), "tiny_kernel(int)", 5_000,
                    {"GRBM_GUI_ACTIVE": 8 * 7_500, "SQ_LDS_IDX_ACTIVE": 1.0})
    assert bench._summarize_lds(str(tmp_path)) == []
    assert bench._summarize_lds(os.path.join(str(tmp_path), "missing")) == []
