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
    start at the 128-row boundary below their group; ragged-K experts above
    1024 tokens run 128-token stages, an even number per expert, from the
    128-token boundary at or below the expert's first padded position, and the
    others go to the exact-group launch (one interleaved step per 8 padded
    tokens)."""
    b = load_bench()
    # one group of 256 rows: a single m-tile, nothing wasted; exact-group launch
    st = b.moe_tile_stats([256], 256, 512, cus=4)
    assert st["raggedM_fwd"]["tiles"] == 2 and st["raggedM_fwd"]["row_waste_frac"] == 0
    assert st["raggedK_wgrad"]["plain_launch"]["experts"] == 0
    assert st["raggedK_wgrad"]["exact_group_launch"]["interleaved_steps_per_tile"] == 256 // 8
    # groups 5, 0, 300: group 2 starts at row 5 (aligned down to 0), so it
    # spans rows 0..304 of its tiles: 2 m-tiles; group 0 needs 1
    st = b.moe_tile_stats([5, 0, 300], 256, 256, cus=2)
    assert st["raggedM_fwd"]["rows_computed"] == 3 * 256
    assert st["raggedM_fwd"]["rows_routed"] == 305
    ex = st["raggedK_wgrad"]["exact_group_launch"]
    assert ex["experts"] == 3 and ex["empty_experts"] == 1 and ex["tokens_routed"] == 305
    assert ex["interleaved_steps_per_tile"] == (32 + 0 + 320) // 8
    # ragged K plain launch: 1100 and 2000 tokens -> ceil32 1120, 2016 -> 9 and
    # 16 stages -> even: 10 and 16; the larger expert's tile goes first
    st = b.moe_tile_stats([1100, 7, 2000], 256, 256, cus=2)
    pl = st["raggedK_wgrad"]["plain_launch"]
    assert pl["experts"] == 2 and pl["tiles"] == 2
    assert pl["tokens_computed"] == (10 + 16) * 128 and pl["tokens_routed"] == 3100
    # workgroup 0: 16 + 1, workgroup 1: 10 + 1
    assert pl["max_over_mean_stages_per_workgroup"] == round(17 / (28 / 2), 4)
    # a group starting off a 128-token boundary reduces from the boundary below:
    # [40, 1250]: group 1 at padded position 64, 64 + 1280 tokens -> 11 stages -> 12
    st = b.moe_tile_stats([40, 1250], 256, 256, cus=1)
    assert st["raggedK_wgrad"]["plain_launch"]["tokens_computed"] == 12 * 128
