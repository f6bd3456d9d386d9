"""CPU checks of the measurement helpers: the rocprofv3 summaries
(`resolution_diffusion_transformer_amd.profiling`) and the bench's reading of
a committed traffic summary, which must only count while the kernel source
still matches the one that was profiled."""
import csv
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from resolution_diffusion_transformer_amd import profiling as P  # noqa: E402


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_counters_sum_instances_within_a_dispatch_then_average_dispatches(tmp_path):
    # kernel A: two dispatches, each reporting FETCH_SIZE from two hardware instances;
    # kernel B: one dispatch
    path = tmp_path / "c.csv"
    _write_csv(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], [
        [1, "A", "FETCH_SIZE", 10.0], [1, "A", "FETCH_SIZE", 30.0],
        [2, "A", "FETCH_SIZE", 50.0], [2, "A", "FETCH_SIZE", 70.0],
        [3, "B", "FETCH_SIZE", 5.0],
    ])
    cs = P.counters(str(path))
    assert sorted(cs["A"]["FETCH_SIZE"]) == [40.0, 120.0]
    assert cs["B"]["FETCH_SIZE"] == [5.0]
    text = P.format_counters(cs)
    line_a = [l for l in text.splitlines() if l.startswith("A ")][0]
    assert "dispatches     2" in line_a and "avg             80.0" in line_a
    assert P.format_counters(cs, only="WRITE_SIZE") == ""


def test_stats_sorted_by_total_time_with_names_shortened(tmp_path):
    path = tmp_path / "s.csv"
    long_name = "void area::(anonymous namespace)::attn_kernel<128, true>(area::(anonymous namespace)::AttnArgs)"
    _write_csv(path, ["Name", "Calls", "TotalDurationNs", "AverageNs"], [
        ["small", 4, 400.0, 100.0],
        [long_name, 2, 6.0e6, 3.0e6],
    ])
    st = P.kernel_stats(str(path))
    assert [s[0] for s in st] == [long_name, "small"]
    text = P.format_stats(st)
    assert "(anonymous namespace)" not in text
    row = text.splitlines()[1].split()
    assert row[-3:] == ["2", "6.000", "3.0000"]


def test_bench_traffic_counts_only_for_the_profiled_source(tmp_path, monkeypatch):
    import bench
    src_dir = tmp_path / "resolution_diffusion_transformer_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / "k_attn.hip"
    src.write_bytes(b"// kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "profiles" / "attn_window_demo_traffic.md"
    prof.write_text(f"# demo\n\n- kernel: attn_kernel\n- k_attn.hip sha256: {sha}\n"
                    "- traffic_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("demo") == 12345.0
    assert bench.measured_traffic("other") is None
    src.write_bytes(b"// kernel source, edited\n")
    assert bench.measured_traffic("demo") is None


def test_dispatches_in_launch_order_per_kernel(tmp_path):
    path = tmp_path / "t.csv"
    _write_csv(path, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], [
        ["blend_kernel(BlendArgs)", 300, 350],
        ["gather_kernel<128>()", 100, 1100],
        ["blend_kernel(BlendArgs)", 50, 80],
        ["attn_kernel<128, true>()", 0, 10],
    ])
    ds = P.dispatches(str(path), ["blend_kernel", "gather_kernel"])
    assert ds["blend_kernel(BlendArgs)"] == [30, 50]
    assert ds["gather_kernel<128>()"] == [1000]
    assert "attn_kernel<128, true>()" not in ds
    text = P.format_dispatches(ds)
    assert "blend_kernel(BlendArgs): 2 dispatches" in text and "0.0" in text
