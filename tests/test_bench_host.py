"""Host-side arithmetic of bench.py: the algorithmic bytes and FLOPs that the
roofline fields divide by, and the rule that a committed HBM-traffic summary
is used only for the kernel source it was measured on.  No GPU needed."""

import importlib.util
import os
import shutil

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_stage_bytes_and_flops_decode_shape(bench):
    from workloads import by_name

    cfg = by_name("decode")
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[:54] = 1  # 54 touched experts
    r = bench.stage_bytes_flops(cfg, counts)
    assert r["touched"] == 54
    # per expert: w13 codes [2I, H/2] + scales [2I, H/16]; w2 codes [H, I/2] + scales [H, I/16]
    w13 = 2 * cfg.I * cfg.H // 2 + 2 * cfg.I * cfg.H // 16
    w2 = cfg.H * cfg.I // 2 + cfg.H * cfg.I // 16
    assert r["gate_up"]["per_expert_bytes"] == w13 == 14_155_776
    assert r["down"]["per_expert_bytes"] == w2 == 7_077_888
    pairs = cfg.T * cfg.k
    x_bytes = cfg.T * (cfg.H // 2 + cfg.H // 16)
    h_bytes = pairs * (cfg.I // 2 + cfg.I // 16)
    assert r["gate_up"]["bytes"] == 54 * w13 + x_bytes + h_bytes == 764_614_656
    assert r["down"]["bytes"] == 54 * w2 + h_bytes + pairs * (cfg.H * 2 + 4)  # FP16 pair rows + row scales
    # FLOPs per pair: 2 H 2I (gate_up) + 2 I H (down)
    assert r["gate_up"]["flops"] + r["down"]["flops"] == pairs * 75_497_472


def test_traffic_summary_only_for_its_own_kernel_source(bench, tmp_path, monkeypatch):
    src = os.path.join(ROOT, "profiles", "ffn_gate_up_decode_pmc.md")
    if not os.path.exists(src):
        pytest.skip("no committed counter summary")
    prof = tmp_path / "profiles"
    prof.mkdir()
    shutil.copy(src, prof / "ffn_gate_up_decode_pmc.md")
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    text = (prof / "ffn_gate_up_decode_pmc.md").read_text()
    current = bench.ffn_source_hash()
    if f"ffn_source_sha256_16: {current}" in text:
        assert bench.read_traffic("ffn_gate_up", "decode") > 0
    # a summary measured on another source is not used
    other = "0" * 16 if current != "0" * 16 else "1" * 16
    lines = [l if not l.startswith("ffn_source_sha256_16:") else f"ffn_source_sha256_16: {other}"
             for l in text.splitlines()]
    (prof / "ffn_gate_up_decode_pmc.md").write_text("\n".join(lines) + "\n")
    assert bench.read_traffic("ffn_gate_up", "decode") is None
    # and a missing summary gives none either
    assert bench.read_traffic("ffn_down", "nonexistent") is None


def test_layer_bytes_and_flops(bench):
    """Whole-layer work of one step: touched experts' weights + router + x + y; FFN + router FLOPs."""
    from workloads import by_name

    cfg = by_name("long_reap")
    counts = np.ones(cfg.E, dtype=np.int64)
    r = bench.layer_bytes_flops(cfg, counts)
    assert r["touched"] == 80
    assert r["flops"] == cfg.pairs * 75_497_472 + 2 * cfg.T * cfg.H * cfg.E
    assert r["bytes"] == 80 * 21_233_664 + cfg.E * cfg.H * 2 + 2 * cfg.T * cfg.H * 2
    # the roofline record: mfma work over seconds against the 2.5 PFLOP/s FP16 peak
    roof = bench._roof("mfma", 2.5e15, 1.0)
    assert roof["unit"] == "TFLOP/s" and abs(roof["frac"] - 1.0) < 1e-12
    roof = bench._roof("hbm", 4e12, 1.0)
    assert roof["unit"] == "GB/s" and abs(roof["frac"] - 0.5) < 1e-12


def test_default_workload_is_the_largest(bench):
    from workloads import CONFIGS

    args = bench.parse_args([])
    assert CONFIGS[args.config].name == "long_reap"
    assert CONFIGS[args.config].T == max(c.T for c in CONFIGS)
    assert bench.main(["--gpus", "2"]) == 2  # several GPUs: refused with a message
