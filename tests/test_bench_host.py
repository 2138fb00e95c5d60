"""Host logic of bench.py on the CPU: the bitwise determinism checker (it
must pass deterministic per-row functions and catch run-to-run noise and
batch dependence) and the traffic figure read from a counter summary (null
once the kernel's sources no longer hash to the recorded value)."""
import time
import pytest
import torch

import bench


def _rows_fn(x):
    # a per-row function: each row's output depends on that row alone
    return lambda idx: [x[idx].sum(dim=1), (x[idx] * 2).to(torch.bfloat16)]


def test_determinism_passes_a_deterministic_per_row_function():
    x = torch.randn(300, 7, generator=torch.Generator().manual_seed(0))
    x[5, 3] = float("nan")          # NaN rows compare by their bits
    f = _rows_fn(x)
    res = bench._determinism(torch, lambda: f(torch.arange(300)), f, 300, device="cpu")
    assert res == {"run_to_run_x3": "pass", "batch_invariance_4splits_1perm": "pass"}


def test_determinism_catches_run_to_run_noise():
    x = torch.randn(64, 3)
    res = bench._determinism(torch, lambda: [x + torch.randn(()) * 1e-7], device="cpu")
    assert res["run_to_run_x3"] == "FAIL"


def test_determinism_catches_batch_dependence():
    x = torch.randn(200, 4, generator=torch.Generator().manual_seed(1))

    def rows(idx):   # depends on how many rows the call holds
        return [x[idx].sum(dim=1) + 1e-3 * len(idx)]

    res = bench._determinism(torch, lambda: rows(torch.arange(200)), rows, 200, device="cpu")
    assert res["run_to_run_x3"] == "pass"
    assert res["batch_invariance_4splits_1perm"] == "FAIL"


def test_determinism_can_be_skipped():
    bench._CHECK_DETERMINISM[0] = False
    try:
        assert "skipped" in bench._determinism(torch, lambda: [torch.zeros(1)], device="cpu")
    finally:
        bench._CHECK_DETERMINISM[0] = True


def test_profile_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    import hashlib
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    (root / "src").mkdir()
    (root / "src" / "k.hip").write_text("kernel source\n")
    (root / "src" / "k.h").write_text("header\n")
    h = hashlib.sha256()
    for f in ("src/k.hip", "src/k.h"):
        h.update((root / f).read_bytes())
    (root / "profiles" / "k_w.md").write_text(
        "# k on w\n\nkernel: k\nsource_files: src/k.hip src/k.h\n"
        f"source_sha256_16: {h.hexdigest()[:16]}\ntraffic_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench._profile_traffic("k_w") == 12345
    with open(root / "src" / "k.h", "a") as fh:    # the kernel's source changes
        fh.write("edited\n")
    assert bench._profile_traffic("k_w") is None
    assert bench._profile_traffic("no_such_summary") is None


def test_sclk_parser(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1800Mhz *\n2: 2400Mhz\n")
    assert bench._read_sclk([str(f)]) == 1800
    f.write_text("S: 2103Mhz *\n")
    assert bench._read_sclk([str(f)]) == 2103
    f.write_text("0: 500Mhz\n")
    assert bench._read_sclk([str(f)]) is None
    assert bench._read_sclk([str(tmp_path / "missing")]) is None


def test_parallel_oracle_covers_every_row():
    seen = []
    bench._POOL["toy"] = lambda lo, hi: sum(range(lo, hi))
    dt = bench._parallel_oracle("toy", 103, 3, 10)
    assert dt >= 0.0
    assert bench._cores() >= 1
    del bench._POOL["toy"], seen


def test_clock_sampler(tmp_path, monkeypatch):
    """The sampler thread reports the DPM level it read."""
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1500Mhz\n2: 2100Mhz *\n")
    monkeypatch.setattr(bench, "_sclk_files", lambda: [str(f)])
    with bench._ClockSampler() as c:
        time.sleep(0.05)
    s = c.summary()
    assert s is not None and s["median_mhz"] == 2100 and s["samples"] >= 1
