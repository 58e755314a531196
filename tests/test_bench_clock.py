"""Host logic of bench.py's clock-adjusted roofline fraction: which clock it takes and when it
refuses one. No GPU: the rules read committed summaries and are tested with stand-ins for them."""
from __future__ import annotations

import json

import bench


def _timeline(tmp_path, sha, modes):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    rec = {"workload": "w", "kernel_sha": sha, "modes": {m: {"sclk_mhz_median": c} for m, c in modes.items()}}
    (prof / "timeline_w.json").write_text(json.dumps(rec))


def test_timeline_clock_preferred_when_its_sources_match(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sha", lambda: "abc")
    monkeypatch.setattr(bench, "load_profile", lambda w, m, key: 1650.0)
    _timeline(tmp_path, "abc", {"causal": 1712.9})
    assert bench.held_clock("w", "causal", 0.02) == (1712.9, "in-kernel timestamps")


def test_stale_timeline_is_ignored(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sha", lambda: "new")
    monkeypatch.setattr(bench, "load_profile", lambda w, m, key: None)
    _timeline(tmp_path, "old", {"causal": 1712.9})
    assert bench.load_timeline("w", "causal") is None
    assert bench.held_clock("w", "causal", 2.0) == (None, None)


def test_counter_clock_only_on_long_launches_and_below_the_top_clock(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))  # no timeline file at all
    monkeypatch.setattr(bench, "kernel_sha", lambda: "abc")
    for clock, launch_ms, want in [(1690.0, 1.8, (1690.0, "GRBM_GUI_ACTIVE")),
                                   (2382.0, 0.037, (None, None)),   # short launch: counter reads high
                                   (2839.0, 0.5, (None, None))]:    # above the top clock: not a clock
        monkeypatch.setattr(bench, "load_profile", lambda w, m, key, c=clock: c)
        assert bench.held_clock("w", "causal", launch_ms) == want


def test_committed_timelines_carry_a_clock_per_mask():
    import workloads
    for name in ("b4h16n1024d128", "gqa_b1h32kv8n16384d128", "b2h16n4096d256_peaked", "z128h8n1024d64_strided"):
        rec = json.load(open(f"{bench.ROOT}/profiles/timeline_{name}.json"))
        modes = {"causal" if c else "non_causal" for c in workloads.WORKLOADS[name].causal_modes}
        # every mask of the workload, plus the static-schedule stamp of launches taking the balanced path
        assert {m for m in rec["modes"] if not m.endswith("_static_schedule")} == modes
        for m in rec["modes"].values():
            assert 500.0 < m["sclk_mhz_median"] <= bench.PEAK_CLOCK_MHZ
            assert len(m["xcd"]["sclk_mhz_median"]) == 8 and len(m["xcd"]["end_us_median"]) == 8
