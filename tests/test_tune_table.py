"""Host logic of the offline tuner: the tuned-table file round-trips and merges."""
from __future__ import annotations

from fp32_sgemm_02_amd import tune


def test_table_round_trip_and_merge(tmp_path):
    path = str(tmp_path / "table.inc")
    first = {(4096, 4096, 4096): {"variant": 1, "tile": 8, "group_m": 0, "gflops": 144287.0},
             (1, 4096, 4096): {"variant": 3, "tile": 0, "group_m": 0, "gflops": 1439.0}}
    tune.write_table(first, path, merge=False)
    assert tune.read_table(path) == first
    # a second tuning run replaces its own shapes and keeps the others
    second = {(4096, 4096, 4096): {"variant": 1, "tile": 2, "group_m": 4, "gflops": 150000.0}}
    tune.write_table(second, path)
    got = tune.read_table(path)
    assert got[(4096, 4096, 4096)]["tile"] == 2 and got[(4096, 4096, 4096)]["group_m"] == 4
    assert got[(1, 4096, 4096)] == first[(1, 4096, 4096)]
    text = open(path).read()
    assert "lookup_tuned" in text and "sentinel" in text
    # the untuned automatic plan winning removes the shape's row
    tune.write_table({(1, 4096, 4096): {"variant": 0, "tile": -1, "group_m": 0, "gflops": 1.0}},
                     path)
    assert (1, 4096, 4096) not in tune.read_table(path)
    assert (4096, 4096, 4096) in tune.read_table(path)


def test_shipped_table_parses_and_names_compiled_tiles():
    import fp32_sgemm_02_amd as sg

    rows = tune.read_table()
    assert (4096, 4096, 4096) in rows
    for shape, r in rows.items():
        assert r["variant"] in (1, 2, 3, 6), shape
        assert 0 <= r["tile"] < sg.tile_count(r["variant"]), f"{shape}: tile {r['tile']} not compiled"
        # the tuned row is what automatic dispatch picks for aligned operands
        M, N, K = shape
        cfg = sg.select(M, N, K, 0x10000, K, 0x20000, N, 0x30000, N)
        assert (cfg.variant, cfg.tile) == (r["variant"], r["tile"]), shape
