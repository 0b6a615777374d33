"""GPU parity of the AWQ W4A16 layer against the CPU oracle, through the C
ABI: the quantizer's codes / scales / zero points bit-exact, exact integer
outputs for on-grid inputs on both kernels (M <= 64 and larger M), and Y
within 1e-2 rms(Y) at the decode sizes M = 1, 16 and the full M = 4608
shape (K 3072, N 12288) on sampled rows."""

import numpy as np
import pytest
import torch

from oracle import awq as OA
from oracle import formats as F
from w4a4_quantized_diffusion_amd import svdq, synth
from tests.gpu_helpers import t_f32, t_x, t_u8, t_bf16_bits, assert_y_close, gm_codes, rm_codes

pytestmark = pytest.mark.gpu


def chunk_rows(a):
    """[N, K/64] -> chunk-major [K/64, N]."""
    return np.ascontiguousarray(np.asarray(a).T)


AWQ = synth.WORKLOADS["awq"]


def awq_layer_to_device(q, s, z, n, k):
    return dict(N=n, K=k, group=64, q=t_u8(gm_codes(OA.pack_nibbles(q))),
                scales=t_bf16_bits(chunk_rows(s)), zeros=t_bf16_bits(chunk_rows(z)))


def test_awq_quantize_weights_bit_exact():
    w = synth.gaussian((400, 1024), 0.02, 0, AWQ, 1)
    w[3, 64:128] = 0.0                      # a zero group: s = 0, z = 0, q = 0
    w[5, :64] = np.abs(w[5, :64])           # min 0
    w[6, :64] = -np.abs(w[6, :64])          # max 0
    q, s, z, packed = OA.quantize_weights(w)
    out = svdq.awq_quantize_weights(t_f32(w))
    torch.cuda.synchronize()
    assert np.array_equal(rm_codes(out["q"].cpu().numpy()), packed), "codes differ"
    sb = out["scales"].cpu().numpy().view(np.uint16).T
    zb = out["zeros"].cpu().numpy().view(np.uint16).T
    assert np.array_equal(sb, F.bf16_bits(s)), "scales differ"
    assert np.array_equal(zb, F.bf16_bits(z)), "zero points differ"


@pytest.mark.parametrize("m", [1, 7, 16, 64, 65, 300])
def test_awq_linear_exact_integers(m):
    """s = 1, integer zero points, small integer X: every product and sum is
    an integer below 2^24, so Y is exact on both kernels (M <= 64 and
    M > 64), ragged N included."""
    g = np.random.default_rng(31)
    k, n = 384, 208
    q = g.integers(0, 16, (n, k)).astype(np.uint8)
    z = g.integers(0, 16, (n, k // 64)).astype(np.float64)
    s = np.ones((n, k // 64))
    x = g.integers(-8, 9, (m, k)).astype(np.float32)
    lay = awq_layer_to_device(q, s, z, n, k)
    y = svdq.awq_linear_w4a16(t_x(x, True), lay, y_dtype=torch.float32)
    ref = OA.linear_w4a16(x, q, s, z)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


def _check_linear(m, k, n, seed, rows=None, ybf16=True):
    x = synth.activations(m, k, seed, AWQ, 0)
    w = synth.gaussian((n, k), 0.02, seed, AWQ, 1)
    b = synth.round_bf16(synth.gaussian((n,), 0.02, seed, AWQ, 2))
    q, s, z, _ = OA.quantize_weights(w)
    lay = awq_layer_to_device(q, s, z, n, k)
    bias = torch.from_numpy(b).to("cuda").to(torch.bfloat16)
    y = svdq.awq_linear_w4a16(t_x(x, True), lay, bias=bias,
                              y_dtype=torch.bfloat16 if ybf16 else torch.float32)
    torch.cuda.synchronize()
    if rows is None:
        rows = np.arange(m)
    y_ref = OA.linear_w4a16(x[rows], q, s, z, b)
    return assert_y_close(y[torch.from_numpy(rows).cuda()], y_ref, ybf16, f"AWQ M={m}")


@pytest.mark.parametrize("m", [1, 16])
def test_awq_linear_decode_sizes(m):
    """The decode-size rows of the AWQ workload: M 1 and 16, K 3072, N 12288."""
    _check_linear(m, 3072, 12288, seed=0, ybf16=True)


@pytest.mark.parametrize("m,k,n", [(3, 192, 48), (77, 640, 144), (300, 1024, 272),
                                   (1, 64, 16), (40, 128, 48), (200, 64, 16)])
def test_awq_linear_ragged(m, k, n):
    _check_linear(m, k, n, seed=2, ybf16=False)


def test_awq_linear_full_size_all_rows():
    """M 4608, K 3072, N 12288: Y within tolerance on every row."""
    _check_linear(4608, 3072, 12288, seed=0, ybf16=True)


@pytest.mark.parametrize("m", [16, 200])
def test_awq_linear_deterministic_and_fully_written(m):
    """Both kernels (M <= 64 and larger M): two runs give the same bits,
    every element of Y is written and nothing past its end."""
    k, n = 1024, 336
    x = synth.activations(m, k, 5, AWQ, 0)
    w = synth.gaussian((n, k), 0.02, 5, AWQ, 1)
    q, s, z, _ = OA.quantize_weights(w)
    lay = awq_layer_to_device(q, s, z, n, k)
    xt = t_x(x, True)
    buf = torch.full((m * n + 4096,), float("nan"), dtype=torch.float32, device="cuda")
    y1 = buf[:m * n].view(m, n)
    svdq.awq_linear_w4a16(xt, lay, Y=y1)
    torch.cuda.synchronize()
    assert not torch.isnan(y1).any(), "unwritten output elements"
    assert torch.isnan(buf[m * n:]).all(), "write past the end of Y"
    y2 = svdq.awq_linear_w4a16(xt, lay, y_dtype=torch.float32)
    assert torch.equal(y1, y2), "two runs differ"
