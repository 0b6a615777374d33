"""GPU parity of the fused GELU input form (the MLP down-projection: the
activation pass applies GELU to its bf16 input first) against the oracle.

The fused step rounds an fp32 GELU value to bf16.  Where the float64 GELU lies
within a few fp32 ulps of a bf16 rounding midpoint, fp32 evaluation may round
either way; both results are correct.  Those elements are found from the
oracle's float64 values alone.  Quantization groups (INT4: 64 along K, NVFP4
blocks of 16) without one are compared bit for bit with the oracle; a group
holding some must equal, bit for bit, the oracle's quantization of one of
the admissible inputs, where each ambiguous element takes either of its two
neighbouring bf16 values.  Y is compared within the layer tolerance
everywhere."""

import itertools

import numpy as np
import pytest
import torch

from oracle import svdq as O
from oracle import nvfp4 as O4
from oracle import formats as F
from w4a4_quantized_diffusion_amd import svdq, synth
from tests.gpu_helpers import (t_f32, t_x, t_u8, t_bf16_bits, layer_to_device, random_int4_layer,
                               assert_y_close, rm_int4, rm_codes, bf16_bits_np)

pytestmark = pytest.mark.gpu


def ambiguous(x):
    """Elements whose fp32 GELU value may round to either neighbouring bf16
    value: the float64 value within 8 + 16 |u| fp32 ulps of a bf16 midpoint
    (u = sqrt(2/pi) (x + 0.044715 x^3); an fp32 evaluation through
    exp(-2u) carries a relative error of a few ulps times |u|)."""
    x = np.asarray(x, dtype=np.float64)
    g32 = F.fl32(O.gelu_tanh(x)).astype(np.float32)
    u = np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)
    margin = 8 + 16 * np.minimum(np.abs(u), 10.0)
    low = (g32.view(np.uint32) & 0xFFFF).astype(np.float64)
    return np.abs(low - 0x8000) <= margin


def neighbours(x):
    """The two bf16 values around the fp32 GELU value of each element (the
    candidates where it lies near their midpoint): truncation of the fp32
    bits and the next bf16 value away from zero."""
    g32 = F.fl32(O.gelu_tanh(np.asarray(x, dtype=np.float64))).astype(np.float32)
    lo = (g32.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    hi = ((g32.view(np.uint32) & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32)
    return lo, hi


def admissible(xg_row, lo, hi, idx, quantize, got, max_enum=12):
    """Whether `got` (the GPU's bytes for one group) equals quantize(v) for
    some admissible input v: xg_row with each element of idx replaced by its
    lo or hi neighbour.  Groups with more than max_enum ambiguous elements
    (none at these sizes) are checked with the first max_enum enumerated and
    the rest at the oracle's choice."""
    idx = np.asarray(idx)[:max_enum]
    for combo in itertools.product((False, True), repeat=len(idx)):
        v = xg_row.copy()
        v[idx] = np.where(combo, hi[idx], lo[idx])
        if quantize(v) == got:
            return True
    return False


def group_mask(amb, width):
    """[rows, K] ambiguity -> [rows, K / width] groups holding one."""
    r, k = amb.shape
    return amb.reshape(r, k // width, width).any(axis=2)


def lr_check(lr_gpu, xg, down, amb):
    """LR within the usual bound, widened by one bf16 step of every ambiguous
    input element."""
    d = np.asarray(down, dtype=np.float64)
    xg64 = xg.astype(np.float64)
    exact = xg64 @ d.T
    sabs = np.abs(xg64) @ np.abs(d).T
    k = xg.shape[1]
    amb_term = (np.abs(xg64) * amb * 2.0 ** -7) @ np.abs(d).T
    got = F.bf16_to_f32(bf16_bits_np(lr_gpu)).astype(np.float64)
    tol = 2.0 ** -8 * np.abs(exact) + 2.0 * k * 2.0 ** -24 * sabs + amb_term
    assert np.all(np.abs(got - exact) <= tol)


def _int4_check(x, lay, rank):
    m, k = x.shape
    d = layer_to_device(lay, rank, lay["q"].shape[0], k)
    codes, scales, lr = svdq.svdq_act_quantize_gelu(t_x(x, True), d)
    torch.cuda.synchronize()
    xg = O.gelu_input(x)
    amb = ambiguous(x)
    gm = group_mask(amb, 64)
    assert gm.mean() < 0.15, f"{gm.mean():.3%} of the groups are ambiguous"
    qx, sa = O.quantize_activations(xg, lay["smooth"])
    got_c = rm_int4(codes.cpu().numpy()).reshape(m, k // 64, 32)
    ref_c = O.pack_int4(qx).reshape(m, k // 64, 32)
    keep = ~gm
    assert np.array_equal(got_c[keep], ref_c[keep]), "codes differ outside ambiguous groups"
    got_s = scales.cpu().numpy().T.view(np.uint32)
    assert np.array_equal(got_s[keep], sa.view(np.uint32)[keep]), "scales differ"
    # every ambiguous group: the GPU's scale and codes are the oracle's for
    # some admissible choice of its ambiguous elements
    lo, hi = neighbours(x)
    smooth = np.asarray(lay["smooth"], dtype=np.float32)

    def q_int4(v, g):
        q, sc = O.quantize_activations(v[None, :], smooth[64 * g:64 * g + 64])
        return O.pack_int4(q).tobytes() + sc.view(np.uint32).tobytes()

    for r, g in zip(*np.nonzero(gm)):
        sl = slice(64 * g, 64 * g + 64)
        got = got_c[r, g].tobytes() + got_s[r, g].tobytes()
        assert admissible(xg[r, sl].copy(), lo[r, sl], hi[r, sl], np.nonzero(amb[r, sl])[0],
                          lambda v: q_int4(v, g), got), f"row {r} group {g}: not admissible"
    if rank:
        lr_check(lr, xg, lay["lora_down"], amb)
    return gm.sum()


def test_act_quantize_gelu_int4():
    s = synth.layer(300, 3072, 16, 0, seed=5, workload="mlp")
    lay = random_int4_layer(64, 3072, 32, seed=5, workload="mlp")
    _int4_check(s["x"], lay, 32)


@pytest.mark.parametrize("rank", [16, 48])
def test_act_quantize_gelu_int4_rows8_and_ragged(rank):
    """M 4100: 8-row workgroups of 4 waves, a ragged last block; rank 16,
    and rank 48 with lora_down prefetched (a LoRA-folded layer's rank)."""
    s = synth.layer(4100, 640, 16, 0, seed=6, workload="mlp")
    lay = random_int4_layer(64, 640, rank, seed=6, workload="mlp")
    _int4_check(s["x"], lay, rank)


def test_act_quantize_gelu_nvfp4():
    m, k = 300, 3072
    x = synth.layer(m, k, 16, 0, seed=7, workload="mlp_fp4")["x"]
    base = random_int4_layer(64, k, 32, seed=7, workload="mlp_fp4")
    xg = O.gelu_input(x)
    ts_x = O4.tensor_scale(np.max(F.fl32(np.abs(xg).astype(np.float64)
                                         * base["smooth"].astype(np.float64))))
    lay = dict(smooth=base["smooth"], lora_down=base["lora_down"], lora_up=base["lora_up"],
               codes=np.zeros((64, k), np.uint8), sbw=np.zeros((64, k // 16), np.uint8),
               ts_w=np.float32(1.0), ts_x=ts_x)
    dd = dict(rank=32, prec=svdq.NVFP4, N=64, K=k, smooth=t_f32(lay["smooth"]),
              lora_down=t_bf16_bits(lay["lora_down"]), lora_up=t_bf16_bits(lay["lora_up"]),
              wcodes=t_u8(np.zeros((k // 64, 64, 32), np.uint8)),
              wscales=t_u8(np.zeros((k // 64, 64, 4), np.uint8)),
              w_tensor_scale=t_f32(np.array([1.0], np.float32)),
              x_tensor_scale=t_f32(np.array([ts_x], np.float32)))
    codes, scales, lr = svdq.svdq_act_quantize_gelu(t_x(x, True), dd)
    torch.cuda.synchronize()
    amb = ambiguous(x)
    gm = group_mask(amb, 16)
    assert gm.mean() < 0.05
    e, sb = O4.quantize_activations(xg, lay["smooth"], ts_x)
    got_c = rm_codes(codes.cpu().numpy())                      # [m, k/2] bytes
    ref_c = O.pack_nibbles(e)
    keep_bytes = np.repeat(~gm, 8, axis=1)                      # 8 bytes per block of 16
    assert np.array_equal(got_c[keep_bytes], ref_c[keep_bytes]), "E2M1 codes differ"
    got_s = scales.cpu().numpy().transpose(1, 0, 2).reshape(m, k // 16)
    assert np.array_equal(got_s[~gm], sb[~gm]), "E4M3 block scales differ"
    # every ambiguous block: admissible (see the module docstring)
    lo, hi = neighbours(x)
    smooth = np.asarray(lay["smooth"], dtype=np.float32)

    def q_fp4(v, b):
        e1, sb1 = O4.quantize_activations(v[None, :], smooth[16 * b:16 * b + 16], ts_x)
        return O.pack_nibbles(e1).tobytes() + sb1.tobytes()

    for r, b in zip(*np.nonzero(gm)):
        sl = slice(16 * b, 16 * b + 16)
        got = got_c[r, 8 * b:8 * b + 8].tobytes() + got_s[r, b:b + 1].tobytes()
        assert admissible(xg[r, sl].copy(), lo[r, sl], hi[r, sl], np.nonzero(amb[r, sl])[0],
                          lambda v: q_fp4(v, b), got), f"row {r} block {b}: not admissible"
    lr_check(lr, xg, lay["lora_down"], amb)


@pytest.mark.parametrize("m,k,n", [(300, 1024, 272), (4608, 12288, 3072)])
def test_linear_gelu_int4(m, k, n):
    """The whole layer on GELU(X): Y within the layer tolerance of the oracle's
    Y for X' = bf16(gelu(X)), on every row (small shape) or sampled rows (the
    MLP down-projection, M 4608 x K 12288 -> N 3072)."""
    x = synth.layer(m, k, 16, 0, seed=8, workload="mlp")["x"]
    lay = random_int4_layer(n, k, 32, seed=8, workload="mlp")
    d = layer_to_device(lay, 32, n, k)
    bias = synth.round_bf16(synth.gaussian((n,), 0.02, 8, synth.WORKLOADS["mlp"], 3))
    y = svdq.svdq_linear_w4a4_gelu(t_x(x, True), d, bias=t_x(bias, True), y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.arange(m) if m <= 512 else np.concatenate(
        [np.random.default_rng(2).choice(m, 16, replace=False), [0, m - 1]])
    y_ref, _ = O.linear_w4a4(O.gelu_input(x[rows]), lay, bias)
    assert_y_close(y[torch.from_numpy(rows).cuda()], y_ref, True, f"GELU layer M{m} K{k} N{n}")


def test_linear_gelu_matches_two_step():
    """The fused layer equals the activation call followed by the GEMM."""
    x = synth.layer(129, 640, 16, 0, seed=9, workload="mlp")["x"]
    lay = random_int4_layer(144, 640, 16, seed=9, workload="mlp")
    d = layer_to_device(lay, 16, 144, 640)
    xt = t_x(x, True)
    y1 = svdq.svdq_linear_w4a4_gelu(xt, d, y_dtype=torch.float32)
    codes, scales, lr = svdq.svdq_act_quantize_gelu(xt, d)
    y2 = svdq.svdq_gemm_w4a4(codes, scales, lr, d, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
