"""The counter and trace reductions behind profiles/ (routed_expert_quantized_amd.pmc),
on small synthetic rocprofv3 CSVs: kernel names, per-dispatch sums and means, the
copy-calibrated byte scaling and the kernel-trace table."""
import csv

import pytest

from routed_expert_quantized_amd import pmc


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def test_short_names_keep_templates_and_drop_arguments():
    assert pmc._short("void moe::k_gemm_dma<0, 2, 0, 6, 3, 64>(unsigned short const*, int)") == \
        "moe::k_gemm_dma<0, 2, 0, 6, 3, 64>"
    assert pmc._short("moe::(anonymous namespace)::k_lora<1>(float*)") == "moe::{anon}::k_lora<1>"
    # parentheses inside template arguments are not the argument list
    assert pmc._short("k<(int)3>(int)") == "k<(int)3>"
    assert pmc._short("plain_kernel") == "plain_kernel"


def test_reduce_sums_each_dispatch_then_averages_over_dispatches(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # a counter read per hardware instance comes as several rows of one dispatch
    p = _write(tmp_path / "c.csv", hdr, [
        [1, "void ka<1>(int)", "FETCH_SIZE", 10.0],
        [1, "void ka<1>(int)", "FETCH_SIZE", 30.0],
        [2, "void ka<1>(int)", "FETCH_SIZE", 20.0],
        [2, "void ka<1>(int)", "FETCH_SIZE", 40.0],
        [3, "kb(float)", "FETCH_SIZE", 7.0],
    ])
    r = pmc.reduce([p])
    assert r["ka<1>"] == {"FETCH_SIZE": 50.0, "dispatches": 2}
    assert r["kb"] == {"FETCH_SIZE": 7.0, "dispatches": 1}
    # dispatch ids of two files do not merge
    r2 = pmc.reduce([p, _write(tmp_path / "d.csv", hdr, [[1, "kb(float)", "FETCH_SIZE", 9.0]])])
    assert r2["kb"] == {"FETCH_SIZE": 8.0, "dispatches": 2}


def test_traffic_scales_by_the_copy_calibration():
    fetch = {"moe::k_gate_up<1>": {"FETCH_SIZE": 100.0, "dispatches": 4},
             "neg_kernel": {"FETCH_SIZE": 512.0, "dispatches": 1}}
    write = {"moe::k_gate_up<1>": {"WRITE_SIZE": 10.0, "dispatches": 4},
             "neg_kernel": {"WRITE_SIZE": 1024.0, "dispatches": 1}}
    r = pmc.traffic(fetch, write, "k_gate_up", "neg", 1024.0 * 1024, sha="abc")
    # the copy read 1 MiB as 512 counter units (2 KiB each) and wrote it as 1024 (1 KiB each)
    assert r["fetch_scale"] == 2048.0 and r["write_scale"] == 1024.0
    assert r["fetch_bytes_per_launch"] == 100.0 * 2048 and r["write_bytes_per_launch"] == 10.0 * 1024
    assert r["bytes_per_launch"] == 100.0 * 2048 + 10.0 * 1024
    assert r["kernel"] == "moe::k_gate_up<1>" and r["kernel_source_sha"] == "abc"
    with pytest.raises(SystemExit):
        pmc.traffic(fetch, write, "k_missing", "neg", 1.0)


def test_traffic_picks_the_most_dispatched_match():
    fetch = {"k<1>": {"FETCH_SIZE": 1.0, "dispatches": 2}, "k<2>": {"FETCH_SIZE": 5.0, "dispatches": 9},
             "neg": {"FETCH_SIZE": 1.0, "dispatches": 1}}
    write = {"k<1>": {"WRITE_SIZE": 1.0, "dispatches": 2}, "k<2>": {"WRITE_SIZE": 3.0, "dispatches": 9},
             "neg": {"WRITE_SIZE": 1.0, "dispatches": 1}}
    r = pmc.traffic(fetch, write, "k<", "neg", 1.0)
    assert r["kernel"] == "k<2>" and r["fetch_bytes_per_launch"] == 5.0


def test_stats_table_orders_by_total_time(tmp_path):
    p = _write(tmp_path / "s.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"], [
        ["void moe::k_small<4>(int)", 10, 10000, 1000, 900, 1200],
        ["void at::native::elementwise_kernel<128, 4, Foo>(int)", 2, 50000, 25000, 20000, 30000],
        ["void moe::k_big<0, 1>(int)", 4, 40000, 10000, 9000, 11000],
    ])
    lines = pmc.stats_table(p).splitlines()
    assert lines[0] == "| kernel | calls | avg (us) | min (us) | max (us) |"
    # other libraries' kernels keep their base name only
    assert lines[2] == "| `at::native::elementwise_kernel<…>` | 2 | 25.00 | 20.00 | 30.00 |"
    assert lines[3] == "| `moe::k_big<0, 1>` | 4 | 10.00 | 9.00 | 11.00 |"
    assert lines[4] == "| `moe::k_small<4>` | 10 | 1.00 | 0.90 | 1.20 |"
    assert len(pmc.stats_table(p, top=1).splitlines()) == 3
