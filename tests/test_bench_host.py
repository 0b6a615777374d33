"""Host-side checks of bench.py (no GPU): the multi-GPU request is refused,
the shader-clock parser reads the sysfs format, and the CPU oracle leg runs
on a tiny layer made by the oracle itself, reporting its fields and a
passing same-run parity check (and a failing one when the 'GPU' output is
perturbed)."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import formats as F  # noqa: E402
from oracle import svdq as O  # noqa: E402
from w4a4_quantized_diffusion_amd import layout, synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_sclk_parser(tmp_path):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("0: 500Mhz\n1: 1800Mhz\n2: 2400Mhz *\n")
    assert bench.read_sclk_mhz(str(p)) == 2400
    p.write_text("S: 2367Mhz *\n")
    assert bench.read_sclk_mhz(str(p)) == 2367
    p.write_text("0: 500Mhz\n")
    assert bench.read_sclk_mhz(str(p)) is None
    assert bench.read_sclk_mhz(str(tmp_path / "missing")) is None


def _ctx(perturb=False):
    M, K, N, R = 96, 128, 64, 16
    s = synth.layer(M, K, N, R, seed=0, workload="flagship")
    xb = F.bf16(s["x"]).astype(np.float32)
    amax = O.act_absmax(xb)
    lay = O.quantize_weights(s["w"], amax, R)
    bias = F.bf16(s["b"]).astype(np.float64)
    y, _ = O.linear_w4a4(xb, lay, bias)
    y = F.bf16(y).astype(np.float32)
    if perturb:
        y[5, 7] += 0.5 * np.sqrt(np.mean(y.astype(np.float64) ** 2))
    qx, sa = O.quantize_activations(xb, lay["smooth"])
    return {"M": M, "K": K, "N": N, "rank": R, "w": s["w"], "amax": amax, "x": xb,
            "bias": bias, "y": y, "act_codes": layout.int4_to_device(O.pack_int4(qx)),
            "act_scales": np.ascontiguousarray(sa.T),
            "wcodes": layout.int4_to_device(lay["wcodes"]),
            "wscales": np.ascontiguousarray(lay["sW"].T), "smooth": lay["smooth"],
            "lora_down_bits": F.bf16_bits(lay["lora_down"]),
            "lora_up_bits": F.bf16_bits(lay["lora_up"])}


def test_cpu_leg_fields_and_parity():
    out = bench.cpu_baseline(_ctx(), 0.2, True)
    assert out["kind"] == "oracle" and out["unit"] == "TOPS" and out["value"] > 0
    assert 1 <= out["cores"] <= out["affinity_cpus"] == len(os.sched_getaffinity(0))
    assert "svd_seconds" in out and "sample" in out
    p = out["parity"]
    assert p["act_codes_bit_exact_all_rows"] and p["act_scales_bit_exact_all_rows"]
    assert p["y_within_tolerance"] and p["y_rows_checked"] >= 1


def test_cpu_leg_flags_a_wrong_output():
    out = bench.cpu_baseline(_ctx(perturb=True), 0.2, False)
    assert out["parity"]["y_rows_checked"] == 96      # the sample covers row 5
    assert not out["parity"]["y_within_tolerance"]
