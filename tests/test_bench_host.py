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


def test_moe_tile_stats_small_cases():
    """Tile accounting of the grouped GEMMs, checked by hand: ragged-M tiles
    start at the 128-row boundary below their group; ragged-K stages are
    128 tokens deep, an even number per group, zero for an empty group."""
    b = load_bench()
    # one group of 256 rows: a single m-tile, nothing wasted
    st = b.moe_tile_stats([256], 256, 512, cus=4)
    assert st["raggedM_fwd"]["tiles"] == 2 and st["raggedM_fwd"]["row_waste_frac"] == 0
    assert st["raggedK_wgrad"]["tokens_computed"] == 256        # 2 stages of 128
    # groups 5, 0, 300: group 2 starts at row 5 (aligned down to 0), so it
    # spans rows 0..304 of its tiles: 2 m-tiles; group 0 needs 1
    st = b.moe_tile_stats([5, 0, 300], 256, 256, cus=2)
    assert st["raggedM_fwd"]["rows_computed"] == 3 * 256
    assert st["raggedM_fwd"]["rows_routed"] == 305
    # ragged K: ceil32 -> 32 and 320 tokens -> 1 and 3 stages -> even: 2 and 4
    assert st["raggedK_wgrad"]["tokens_computed"] == (2 + 0 + 4) * 128
    assert st["raggedK_wgrad"]["tiles"] == 3
    # the largest group's tile goes first: workgroup 0 gets 4 + 1 and 0 + 1
    # (the empty group), workgroup 1 gets 2 + 1
    assert st["raggedK_wgrad"]["max_over_mean_stages_per_workgroup"] == round(6 / (9 / 2), 4)
