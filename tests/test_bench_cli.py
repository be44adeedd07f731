"""bench.py's command line without a GPU: it measures one GPU only and says so."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_trace_reader_takes_the_main_instantiation_and_checks_the_sources(tmp_path, monkeypatch):
    """The bench reads a kernel's traced average from the committed trace only
    while its "kernel source sha" matches, and of several instantiations of one
    kernel takes the first row (the table is sorted by total time)."""
    sys.path.insert(0, ROOT)
    import bench
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "kernel_trace_demo.md").write_text(
        "# demo\n\nkernel source sha: abc123\n\n| kernel | calls | avg (us) | min (us) | max (us) |\n|---|---|---|---|---|\n"
        "| `moe::k_gemm_dma<1, 1, 0, 1, 2, 128>` | 10 | 95.00 | 90.00 | 99.00 |\n"
        "| `moe::k_gemm_dma<1, 1, 1, 1, 2, 64>` | 10 | 48.00 | 45.00 | 50.00 |\n"
        "| `moe::k_gemm_dma<1, 1, 0, 4, 2, 64>` | 2 | 30.00 | 29.00 | 31.00 |\n"
        "| `moe::k_gate_up_t1<0, 1, 1, 1, 1, 4, true>` | 5 | 7.40 | 7.00 | 8.00 |\n"
        "| `moe::k_gate_up_t1<0, 1, 1, 1, 2, 4, true>` | 1 | 9.00 | 9.00 | 9.00 |\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench.trace_kernel_us("demo", "abc123")
    assert got == {"gemm_gate_up": 95.0, "gemm_down": 48.0, "gate_up": 7.4}
    assert bench.trace_kernel_us("demo", "fff000") is None
    assert bench.trace_kernel_us("absent", "abc123") is None
