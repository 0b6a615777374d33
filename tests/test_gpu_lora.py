"""GPU parity of the LoRA fold (svdq_fold_lora) against the oracle, through
the C ABI: the folded factors bit-exact (B scaled in fp32 and rounded to
bf16 on both sides), and the INT4 / NVFP4 layers run at the longer rank
within the Y tolerance of the unfolded layers."""

import numpy as np
import pytest
import torch

from oracle import svdq as O
from oracle import nvfp4 as O4
from oracle import formats as F
from w4a4_quantized_diffusion_amd import svdq, synth
from tests.gpu_helpers import (t_x, t_f32, t_bf16_bits, layer_to_device, bf16_bits_np,
                               assert_y_close)
from tests.test_gpu_nvfp4 import nv_layer_to_device

pytestmark = pytest.mark.gpu


def _adapter(n, k, r_lora, seed):
    a, b = synth.lora_adapter(n, k, r_lora, seed)
    return a.astype(np.float64), b.astype(np.float64)


@pytest.mark.parametrize("n,k,rank,r_lora,scale", [
    (272, 192, 32, 16, 1.0),      # no padding, B copied bit for bit
    (144, 640, 16, 5, 0.8),       # padding 11, B rounded after scaling
    (48, 64, 0, 7, -2.5),         # no base branch
    (1000, 128, 240, 16, 0.3),    # the longest rank the kernels take
])
def test_fold_lora_bit_exact(n, k, rank, r_lora, scale):
    print(f"fold_lora n={n} k={k} rank={rank} r_lora={r_lora}", flush=True)
    g = np.random.default_rng(rank + r_lora)
    down = synth.round_bf16(g.standard_normal((rank, k)) * 0.1).astype(np.float64)
    up = synth.round_bf16(g.standard_normal((n, rank)) * 0.1).astype(np.float64)
    a, b = _adapter(n, k, r_lora, 1)
    d = dict(N=n, K=k, rank=rank, lora_down=t_bf16_bits(down), lora_up=t_bf16_bits(up))
    out = svdq.svdq_fold_lora(d, t_bf16_bits(a), t_bf16_bits(b), scale)
    torch.cuda.synchronize()
    d2, u2, r_new = O.fold_lora(down if rank else None, up if rank else None, a, b, scale)
    assert out["rank"] == r_new
    assert np.array_equal(bf16_bits_np(out["lora_down"]), F.bf16_bits(d2))
    assert np.array_equal(bf16_bits_np(out["lora_up"]), F.bf16_bits(u2))


@pytest.mark.parametrize("m,k,n,rank,r_lora", [(300, 512, 272, 32, 16), (77, 192, 48, 0, 9)])
def test_int4_linear_with_folded_lora(m, k, n, rank, r_lora):
    print(f"int4 linear + lora {m}x{k}x{n} rank={rank} r_lora={r_lora}", flush=True)
    s = synth.layer(m, k, n, rank, seed=4, workload="attn")
    lay = O.quantize_weights(s["w"], O.act_absmax(s["x"]), rank)
    a, b = _adapter(n, k, r_lora, 2)
    d = svdq.svdq_fold_lora(layer_to_device(lay, rank, n, k), t_bf16_bits(a), t_bf16_bits(b),
                            0.75)
    d2, u2, r_new = O.fold_lora(lay["lora_down"] if rank else None,
                                lay["lora_up"] if rank else None, a, b, 0.75)
    lay2 = dict(lay, lora_down=d2, lora_up=u2)
    bias = synth.round_bf16(s["b"])
    y_ref, _ = O.linear_w4a4(s["x"], lay2, bias)
    for ybf16 in (False, True):
        y = svdq.svdq_linear_w4a4(t_x(s["x"], True), d, bias=t_x(bias, True),
                                  y_dtype=torch.bfloat16 if ybf16 else torch.float32)
        assert_y_close(y, y_ref, ybf16, f"folded rank {r_new}")
    # the adapter really changed the output
    y0, _ = O.linear_w4a4(s["x"], lay, bias)
    assert np.abs(y_ref - y0).max() > 0.1 * np.sqrt(np.mean(y_ref ** 2))


def test_nvfp4_linear_with_folded_lora():
    m, k, n, rank, r_lora = 130, 256, 144, 16, 16
    print(f"nvfp4 linear + lora {m}x{k}x{n} rank={rank} r_lora={r_lora}", flush=True)
    s = synth.layer(m, k, n, rank, seed=5, workload="attn")
    lay = O4.quantize_weights(s["w"], O.act_absmax(s["x"]), rank)
    a, b = _adapter(n, k, r_lora, 3)
    d = svdq.svdq_fold_lora(nv_layer_to_device(lay, rank, n, k), t_bf16_bits(a),
                            t_bf16_bits(b), 1.0)
    d2, u2, _ = O.fold_lora(lay["lora_down"], lay["lora_up"], a, b, 1.0)
    bias = synth.round_bf16(s["b"])
    y_ref, _ = O4.linear_nvfp4(s["x"], dict(lay, lora_down=d2, lora_up=u2), bias)
    y = svdq.svdq_linear_w4a4(t_x(s["x"], True), d, bias=t_x(bias, True))
    assert_y_close(y, y_ref, False, "nvfp4 folded")
