"""Host-side logic of bench.py (no GPU): the roofline's HBM traffic comes from
the committed counter summary only while the GEMM source is unchanged."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_measured_traffic_reads_summary_of_current_source(tmp_path):
    b = load_bench()
    digest = b.source_digest(b.GEMM_SRC)
    (tmp_path / "k__hbm_traffic.md").write_text(
        "# x\n\n- HBM bytes per launch: 1234\n- kernel source sha256[:16]: " + digest + "\n")
    (tmp_path / "old__hbm_traffic.md").write_text(
        "# x\n\n- HBM bytes per launch: 99\n- kernel source sha256[:16]: 0000000000000000\n")
    b.PROFILE_DIR = str(tmp_path)
    assert b.measured_traffic("k") == 1234
    assert b.measured_traffic("old") is None        # profiled with another kernel source
    assert b.measured_traffic("missing") is None


def test_committed_profiles_name_the_profiled_source():
    b = load_bench()
    path = os.path.join(ROOT, "profiles", "moe_gemm_wgrad_raggedK__hbm_traffic.md")
    text = open(path).read()
    assert "kernel source sha256[:16]: " in text and "HBM bytes per launch: " in text
