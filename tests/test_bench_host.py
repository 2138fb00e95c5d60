"""Host logic of bench.py on the CPU: the bitwise determinism checker (it
must pass deterministic per-row functions and catch run-to-run noise and
batch dependence) and the traffic figure read from a counter summary (null
once the kernel's sources no longer hash to the recorded value)."""
import os
import shutil

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
    name = "bf16_hist_rows_qwen3_logits_4096x151936"
    assert isinstance(bench._profile_traffic(name), int)    # committed summary matches
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    shutil.copy(os.path.join(bench.ROOT, "profiles", name + ".md"), root / "profiles")
    text = (root / "profiles" / (name + ".md")).read_text()
    files = [ln.split(":", 1)[1].split() for ln in text.splitlines()
             if ln.startswith("source_files:")][0]
    for f in files:
        (root / f).parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, f), root / f)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench._profile_traffic(name) == int(
        [ln.split(":")[1] for ln in text.splitlines() if ln.startswith("traffic_bytes")][0])
    with open(root / files[0], "a") as fh:     # the kernel's source changes
        fh.write("\n// edited\n")
    assert bench._profile_traffic(name) is None
    assert bench._profile_traffic("no_such_summary") is None
