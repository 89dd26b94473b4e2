"""Host-side pieces of bench.py (no GPU): the refusal of more than one GPU,
the algorithmic byte counts, and the counted-source hash that keys the stored
HBM counters (bench.py reports no traffic once the counted code changes)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_source_hash_ignores_comments_and_layout_but_not_code():
    src = 'int f(int a) {  // doubles\n  /* no side effects */ return 2 * a; }\nconst char *s = "// kept";\n'
    base = bench._code_only("k.hip", src)
    assert base == 'int f(int a) { return 2 * a; } const char *s = "// kept";'
    assert bench._code_only("k.hip", src.replace("doubles", "twice")) == base
    assert bench._code_only("k.hip", src.replace("  return", "\n\n    return")) == base
    assert bench._code_only("k.hip", src.replace("2 * a", "3 * a")) != base
    assert bench._code_only("k.hip", src.replace('"// kept"', '"// changed"')) != base
    # other files are hashed as they are
    assert bench._code_only("build.py", "x = 1  # note\n") == "x = 1  # note\n"


def test_algorithmic_bytes_of_the_100k_session():
    b = bench.compaction_bytes(288, 100000, 128, 4, 32, 2048)
    # K (T*d bf16) + the group's window queries + fp32 scores, per row
    assert b["kvc_score"] == 288 * (100000 * 128 * 2 + 4 * 32 * 128 * 2 + 100000 * 4)
    # B keys and values read and written, input and output positions
    assert b["kvc_compact_rerotate"] == 288 * (4 * 2048 * 128 * 2 + 2048 * 8)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_pipeline_call_times_are_medians_over_the_runs(monkeypatch):
    """One run delayed on the host (here the second call of the first run) does
    not move a call's figure: each call takes the median over the runs."""
    import torch
    from budgeted_retention_amd import pipelines

    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t

    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    timer = pipelines.CallTimer()
    runs = [{"score": 3.0, "select": 9.0}, {"score": 3.2, "select": 0.1}, {"score": 2.8, "select": 0.12}]
    for r in runs:
        for name in ("score", "select"):
            timer.events.append((name, Ev(0.0), Ev(r[name])))
    med = timer.median_step_ms(3)
    assert med == {"score": 3.0, "select": 0.12}
    with pytest.raises(ValueError):
        timer.median_step_ms(4)


def test_shader_clock_reads_the_current_level(tmp_path, monkeypatch):
    """The clock comes from the driver's table: the level marked '*'; the
    device's own PCI path is tried first, then every card; None when absent."""
    import glob as _glob

    class Props:
        pci_domain_id, pci_bus_id, pci_device_id = 0xfff0, 0x75, 0   # a PCI path no machine has

    table = tmp_path / "pp_dpm_sclk"
    table.write_text("0: 500Mhz \n1: 1800Mhz \n2: 2400Mhz *\n")
    monkeypatch.setattr(_glob, "glob", lambda pattern: [str(table)] if "drm" in pattern else [])
    assert bench.shader_clock(Props()) == "2400Mhz"
    table.write_text("0: 500Mhz \n1: 1800Mhz \n")
    assert bench.shader_clock(Props()) is None
    monkeypatch.setattr(_glob, "glob", lambda pattern: [])
    assert bench.shader_clock(Props()) is None
