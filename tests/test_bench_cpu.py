"""Host-side checks of bench.py's reporting logic (no GPU): the one-GPU guard,
the classification of kernel records, the Winograd forms' MFMA fractions and
the rule that counter-derived HBM traffic is reported only for the kernel
source it was measured on."""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line for a configuration that was not measured


@pytest.mark.parametrize("name, fam", [
    ("conv3x3_wino4<16,plain>", "conv3x3_wino4"),
    ("conv3x3_wino4<16,up2x>", "conv3x3_wino4"),
    ("conv3x3_wino<16,plain,res>", "conv3x3_wino"),
    ("conv3x3_mfma<32,denorm>", "conv3x3_mfma"),
    ("conv3x3_direct", ""),          # conv_out: VALU kernel, not counted with the MFMA convs
    ("gemm_mfma", ""),
    ("groupnorm_silu", ""),
])
def test_conv_family(name, fam):
    assert bench.conv_family(name) == fam
    assert bench.is_conv3x3(name) == (fam != "")


def test_mfma_fractions():
    # products executed per direct-conv multiply: F(4x4) 36 of 144 points (25
    # distinct on a nearest-x2 input), F(2x2) 16 of 36 (9), direct forms all
    assert bench.mfma_fraction("conv3x3_wino4<16,plain>") == 36 / 144
    assert bench.mfma_fraction("conv3x3_wino4<16,plain,res>") == 36 / 144
    assert bench.mfma_fraction("conv3x3_wino4<16,up2x>") == 25 / 144
    assert bench.mfma_fraction("conv3x3_wino<16,plain>") == 16 / 36
    assert bench.mfma_fraction("conv3x3_wino<16,up2x>") == 9 / 36
    assert bench.mfma_fraction("conv3x3_mfma<32,plain>") == 1.0
    assert bench.mfma_fraction("gemm_mfma") == 1.0


def _summary(path, kernel, sha, traffic=123456789):
    with open(path, "w") as f:
        f.write(f"# counters\n\ntraffic_bytes_per_launch: {traffic}\nkernel: {kernel}\nkernel_source_sha256: {sha}\n")


def test_counter_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    prof = tmp_path / "profiles"
    csrc.mkdir()
    prof.mkdir()
    src = b"// kernel source as profiled\n"
    (csrc / "conv_wino4.hip").write_bytes(src)
    sha = hashlib.sha256(src).hexdigest()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    summary = prof / "conv3x3_wino4_decode1024_hbm_counters.md"
    _summary(summary, "conv3x3_wino4<16,plain>", sha)

    assert bench.counter_traffic("conv3x3_wino4<16,plain>", "decode1024") == 123456789.0
    # another workload, another instantiation or a non-conv kernel: not measured
    assert bench.counter_traffic("conv3x3_wino4<16,plain>", "decode256") is None
    assert bench.counter_traffic("conv3x3_wino4<16,plain,res>", "decode1024") is None
    assert bench.counter_traffic("gemm_mfma", "decode1024") is None
    # the source changed since the counters were taken: stale, so null
    (csrc / "conv_wino4.hip").write_bytes(src + b"// edited\n")
    assert bench.counter_traffic("conv3x3_wino4<16,plain>", "decode1024") is None
    # no summary at all
    summary.unlink()
    assert bench.counter_traffic("conv3x3_wino4<16,plain>", "decode1024") is None


def test_committed_counter_summary_names_its_kernel():
    """The committed summary for the dominant kernel carries the fields bench.py
    reads, and its source hash is a SHA-256 digest."""
    path = os.path.join(ROOT, "profiles", "conv3x3_wino4_decode1024_hbm_counters.md")
    vals = {}
    for line in open(path).read().splitlines():
        key, _, val = line.partition(": ")
        vals[key] = val.strip()
    assert vals["kernel"].startswith("conv3x3_wino4<")
    assert float(vals["traffic_bytes_per_launch"]) > 0
    assert len(vals["kernel_source_sha256"]) == 64
    int(vals["kernel_source_sha256"], 16)


def test_roofline_of_a_winograd_kernel_counts_executed_products():
    # 14 launches of the F(4x4) conv at 270.58 GFLOP of direct-conv work in
    # 0.807 ms each: the MFMA pipes run 36/144 of those multiplies, so the
    # fraction of the FP32 MFMA peak is 0.533, never above 1
    k = {"ms": 14 * 0.807, "flops": 14 * 270.582939648e9, "bytes": 14 * 4.84e8, "n": 14}
    r = bench.roofline("conv3x3_wino4<16,plain>", k, 1, "decode256")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["flops_per_launch"] == pytest.approx(270.582939648e9 * 36 / 144)
    assert r["achieved"] == pytest.approx(r["flops_per_launch"] / 0.807e-3 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 157.3)
    assert 0.5 < r["frac"] <= 1.0
    assert r["direct_equivalent_tflops"] == pytest.approx(r["achieved"] * 4)
    assert r["launches_per_step"] == 14


@pytest.mark.parametrize("name", ["conv3x3_wino4<16,plain>", "conv3x3_wino4<16,up2x>", "conv3x3_wino<16,plain>",
                                  "conv3x3_mfma<32,plain>", "gemm_mfma"])
def test_roofline_fraction_never_exceeds_one_at_the_peak(name):
    # a launch that executes exactly the peak's worth of MFMA work in its time
    # sits at frac 1, whatever its direct-conv count
    f = bench.mfma_fraction(name)
    ms = 1.0
    direct = 157.3e12 * ms / 1e3 / f
    r = bench.roofline(name, {"ms": ms, "flops": direct, "bytes": 1.0, "n": 1}, 1, "decode256")
    assert r["frac"] == pytest.approx(1.0)


def test_roofline_of_a_memory_bound_kernel():
    r = bench.roofline("groupnorm_silu", {"ms": 2.0, "flops": 0.0, "bytes": 2 * 4e9, "n": 2}, 1, "decode1024")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4e9 / 1e-3 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)


def test_decode_flops_follow_the_architecture():
    # per-conv 2 Cin Cout k^2 H W plus attention 8 N c^2 + 4 N^2 c, summed
    # over the chain; the 1024x1024 total equals the one the decoder's own
    # per-launch records add up to (10.472 TFLOP)
    import vaegen
    p = vaegen.decoder_params(0)
    assert bench.decode_flops(p, 128, 128) == 10472204009472.0
    n, c = 32 * 32, 512
    attn = 8.0 * n * c * c + 4.0 * n * n * c
    assert bench.decode_flops(p, 32, 32) - attn == pytest.approx(618.0e9, rel=1e-3)
    # conv FLOPs scale with the latent area
    a8 = bench.decode_flops(p, 8, 8) - (8.0 * 64 * c * c + 4.0 * 64 * 64 * c)
    assert bench.decode_flops(p, 32, 32) - attn == pytest.approx(16 * a8)


def test_form_fractions():
    assert bench.form_fraction("winograd_4x4") == 36 / 144
    assert bench.form_fraction("winograd_4x4", upsample=True) == 25 / 144
    assert bench.form_fraction("winograd_2x2") == 16 / 36
    assert bench.form_fraction("implicit_gemm") == 1.0
