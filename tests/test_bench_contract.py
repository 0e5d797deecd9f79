"""CPU checks of bench.py's command-line contract that need no GPU: more than one GPU is refused with a
message and a non-zero status before anything touches a device, and the headline workload is named."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 2 is not supported" in r.stderr and "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_workloads_are_chosen_by_name():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "3"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0 and "invalid choice" in r.stderr


def test_row_summary_stays_short():
    """The headline record carries one short entry per row; with every row kind present (values of the
    sizes a run prints) the summary stays well under the 4 KB the whole record is kept within."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    call = {"us": 1.0, "GB/s": 1.0}
    two = {"us_per_step": 193.99, "GB/s": 5632.3, "calls": {"quantize": call, "reduce_shard": call, "gather": call}}
    share = dict(two, mode="P")
    extra = {
        "two_step_llama3-8b-decode": two, "share_llama3-70b-prefill": share, "share_llama3-8b-decode": share,
        "norm_first_llama3-70b-prefill": dict(two, share=share), "norm_first_llama3-8b-decode": dict(two, share=share),
        "self_sync_slots": {"pass1_us": 10.64, "pass1_GB/s": 3329.1, "retry_us": 8.46, "pending_blocks": 1263,
                            "pass1_nocount_us": 8.8, "pass1_nocount_GB/s": 4000.0},
        "self_sync_allgather": {"by_payload": {t: {"pass1_us": 22.43, "pass1_GB/s": 4615.2, "retry_us": 15.46}
                                               for t in ("bf16_shards", "int8_prefill_messages")}},
        "tokenweave_reduce_rmsnorm": {"both_halves_us": 251.4, "both_halves_GB/s": 5872.8,
                                      "max_workgroups_sweep": {"rows": {"overlap_makespan_us": 497.7,
                                                                        "serial_us": 596.5}}},
        "two_half_layer": {"by_T": {"8192": {"pipelined_us": 1070.7, "serial_halves_us": 1129.8,
                                             "unsplit_us": 1218.0}}},
        "readiness_encodings": {"choice_matches_fastest_measured": "26/33",
                                "committed_table": {"points": 33, "fastest": 25, "mean_pct": 0.4, "max_pct": 4.7}},
        "warm_caches": {"us_per_step": 180.0, "GB/s": 6000.0},
    }
    s = bench.row_summary(extra)
    assert len(s) == len(extra) + 1  # the all-gather row splits into its two payloads
    assert len(json.dumps(s)) < 2500


def test_profile_commands_name_the_tables_they_came_from():
    """The profile summaries print the rocprofv3 command of each table they read: output directory and
    name come from the table's own path, whatever directory the run wrote to."""
    import pytest
    sys.path.insert(0, ROOT)
    import bench
    assert bench._rp_out("out/st_x/st_kernel_stats.csv") == "-d out/st_x -o st"
    assert bench._rp_out("a/b/pmc1_counter_collection.csv") == "-d a/b -o pmc1"
    with pytest.raises(ValueError):
        bench._rp_out("a/b/st_kernel_trace.csv")
