"""GPU parity of the INT4 SVDQuant path against the CPU oracle, through the
C ABI: activation codes / scales bit-exact, LR within one bf16 step, exact
integer group sums (unit-scale mode), Y within 1e-2 rms(Y), the offline
quantizer's smoothing / residual / codes bit-exact for a given low-rank
split, and full-size runs in the benchmark's launch configuration checked on
sampled rows."""

import numpy as np
import pytest
import torch

from oracle import svdq as O
from oracle import formats as F
from w4a4_quantized_diffusion_amd import svdq, synth
from tests.gpu_helpers import (t_f32, t_x, t_u8, t_bf16_bits, layer_to_device,
                               random_int4_layer, bf16_bits_np, assert_lr_close, assert_y_close,
                               gm_int4, rm_int4, gm_scales, degenerate_activations)

pytestmark = pytest.mark.gpu


def _oracle_layer(w, x, rank):
    return O.quantize_weights(w, O.act_absmax(x), rank)


def _check_act(x_np, lay, rank, bf16):
    m, k = x_np.shape
    d = layer_to_device(lay, rank, lay["q"].shape[0], k)
    codes, scales, lr = svdq.svdq_act_quantize(t_x(x_np, bf16), d)
    torch.cuda.synchronize()
    qx, sa = O.quantize_activations(x_np, lay["smooth"])
    assert np.array_equal(rm_int4(codes.cpu().numpy()), O.pack_int4(qx)), "activation codes differ"
    assert np.array_equal(scales.cpu().numpy().T.view(np.uint32), sa.view(np.uint32)), "scales differ"
    if rank:
        mism = assert_lr_close(lr, x_np, lay["lora_down"], "LR")
        assert mism <= 0.01 * lr.numel(), f"{mism} LR entries differ from the oracle's bits"
        return mism
    return 0


def test_act_quant_small_workload_fp32():
    s = synth.small()
    lay = _oracle_layer(s["w"], s["x"], s["rank"])
    _check_act(s["x"], lay, s["rank"], bf16=False)


@pytest.mark.parametrize("m", [1, 100, 257])
def test_act_quant_bf16_ragged_rows(m):
    s = synth.layer(m, 3072, 256, 32, seed=1, workload="attn")
    lay = _oracle_layer(s["w"], s["x"], 32)
    _check_act(s["x"], lay, 32, bf16=True)


@pytest.mark.parametrize("rank", [0, 32, 48])
def test_act_quant_large_m(rank):
    """M 4104 (a ragged tail past 16 x 256 rows): 8-row workgroups, of 4 waves
    with the low-rank branch, lora_down prefetched at ranks 32 and 48."""
    s = synth.layer(4104, 3072, 64, rank, seed=8, workload="attn")
    lay = _oracle_layer(s["w"], s["x"], rank)
    _check_act(s["x"], lay, rank, bf16=True)


def test_act_quant_half_integer_ties():
    """Group amax 14 (scale 2, exact reciprocal) and 21 (scale 3, inexact
    reciprocal): every quotient that is a half-integer 0.5 ... 6.5, the values
    one ulp on either side of it, both signs, so that each tie and each
    near-tie is decided by the correctly rounded quotient (the reciprocal
    alone would misjudge some for scale 3).  Codes and scales must match the
    oracle bit for bit; -0.5 and the values just above it give code 0."""
    k, m = 512, 16
    halves = np.arange(7, dtype=np.float32) + np.float32(0.5)
    x = np.zeros((m, k), np.float32)
    for r in range(m):
        for g in range(k // 64):
            s = np.float32(2.0 if (r + g) % 2 else 3.0)
            z = halves * s
            vals = np.concatenate([z, np.nextafter(z, np.float32(0)), np.nextafter(z, np.float32(99))])
            vals = np.concatenate([vals, -vals])
            x[r, 64 * g] = 7 * s if (r + g) % 3 else -7 * s
            for i in range(1, 64):
                x[r, 64 * g + i] = vals[(r * 5 + g * 11 + i) % vals.size]
    lay = dict(smooth=np.ones(k, np.float32), q=np.zeros((16, k), np.int8),
               wcodes=np.zeros((16, k // 2), np.uint8), sW=np.ones((16, k // 64), np.float32),
               lora_down=None, lora_up=None)
    _check_act(x, lay, 0, bf16=False)


def test_act_quant_degenerate_inputs():
    """All-zero rows and groups (scale 0, codes 0), constant groups, subnormal
    and huge values, scales that underflow or are subnormal (the exact
    division path): codes and scales bit-exact against the oracle."""
    x = degenerate_activations(seed=3)
    k = x.shape[1]
    lay = dict(smooth=np.ones(k, np.float32), q=np.zeros((16, k), np.int8),
               wcodes=np.zeros((16, k // 2), np.uint8), sW=np.ones((16, k // 64), np.float32),
               lora_down=None, lora_up=None)
    _check_act(x, lay, 0, bf16=False)


@pytest.mark.parametrize("m", [100, 4096, 4608])
def test_act_quant_scales_over_the_exponent_range(m):
    """Group maxima spread over the whole fp32 range (each group's values a
    normal sample times 2^e, e in [-135, 122], times a non-trivial fp32
    smoothing factor): the scale fl32(amax / 7) and the codes, bit for bit,
    from the smallest subnormal scales to the largest, including the ranges
    below 2^-100 and above 2^100 where the kernels divide directly."""
    k = 128
    g = np.random.default_rng(17)
    e = g.integers(-135, 123, size=(m, k // 64))
    x = g.normal(size=(m, k)) * np.exp2(np.repeat(e, 64, axis=1))
    x = x.astype(np.float32)
    smooth = g.uniform(0.5, 2.0, size=k).astype(np.float32)
    lay = dict(smooth=smooth, q=np.zeros((16, k), np.int8),
               wcodes=np.zeros((16, k // 2), np.uint8), sW=np.ones((16, k // 64), np.float32),
               lora_down=None, lora_up=None)
    _check_act(x, lay, 0, bf16=False)


def test_gemm_unit_scale_exact_integers():
    """rank 0, all scales 1, no bias, fp32 out: Y is the exact integer dot
    product of the codes (below 2^24, so exact in fp32)."""
    g = np.random.default_rng(7)
    m, k, n = 130, 320, 208
    qx = g.integers(-7, 8, (m, k)).astype(np.int8)
    qw = g.integers(-7, 8, (n, k)).astype(np.int8)
    qx[0, :] = 7
    qw[0, :] = -7                                    # extreme sums -49*k
    ones_a = torch.ones((k // 64, m), dtype=torch.float32, device="cuda")
    lay = dict(rank=0, prec=0, N=n, K=k, wcodes=t_u8(gm_int4(O.pack_int4(qw))),
               wscales=torch.ones((k // 64, n), dtype=torch.float32, device="cuda"),
               lora_up=None, w_tensor_scale=None, x_tensor_scale=None)
    y = svdq.svdq_gemm_w4a4(t_u8(gm_int4(O.pack_int4(qx))), ones_a, None, lay)
    ref = sum(O.group_int_products(qx, qw, gi) for gi in range(k // 64))
    assert np.array_equal(y.cpu().numpy(), ref.astype(np.float32))


def test_gemm_single_nonzero_group():
    """Only group 2 non-zero, per-row/column power-of-two scales: the output is
    exactly sA sW I_2."""
    g = np.random.default_rng(8)
    m, k, n = 64, 256, 64
    qx = np.zeros((m, k), np.int8)
    qw = np.zeros((n, k), np.int8)
    qx[:, 128:192] = g.integers(-7, 8, (m, 64))
    qw[:, 128:192] = g.integers(-7, 8, (n, 64))
    sa = np.ldexp(1.0, g.integers(-8, 8, (m, k // 64))).astype(np.float32)
    sw = np.ldexp(1.0, g.integers(-8, 8, (n, k // 64))).astype(np.float32)
    lay = dict(rank=0, prec=0, N=n, K=k, wcodes=t_u8(gm_int4(O.pack_int4(qw))),
               wscales=t_f32(gm_scales(sw)), lora_up=None, w_tensor_scale=None,
               x_tensor_scale=None)
    y = svdq.svdq_gemm_w4a4(t_u8(gm_int4(O.pack_int4(qx))), t_f32(gm_scales(sa)), None, lay)
    ref = sa[:, 2:3].astype(np.float64) * sw[:, 2].astype(np.float64)[None, :] * \
        O.group_int_products(qx, qw, 2)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("ybf16", [False, True])
def test_linear_small_workload(ybf16):
    s = synth.small()
    lay = _oracle_layer(s["w"], s["x"], s["rank"])
    d = layer_to_device(lay, s["rank"], 1024, 1024)
    y = svdq.svdq_linear_w4a4(t_x(s["x"], False), d, bias=t_f32(s["b"]),
                              y_dtype=torch.bfloat16 if ybf16 else torch.float32)
    y_ref, _ = O.linear_w4a4(s["x"], lay, s["b"])
    assert_y_close(y, y_ref, ybf16, "small workload")


@pytest.mark.parametrize("m,k,n,rank", [(77, 192, 48, 16), (300, 1024, 272, 32),
                                        (129, 640, 144, 0), (5, 3072, 400, 48),
                                        (1, 64, 16, 0), (300, 64, 272, 32), (33, 128, 48, 16),
                                        (130, 256, 80, 64), (70, 512, 272, 256)])
def test_linear_ragged_shapes(m, k, n, rank):
    """Ragged M / N tiles; K = 64 and 128 leave most waves of the activation
    kernel without a K-group and run the GEMM with one or two groups; ranks
    64 and 256 take the epilogue's low-rank loads in two and eight batches."""
    s = synth.layer(m, k, n, rank, seed=3, workload="attn")
    lay = _oracle_layer(s["w"], s["x"], rank)
    d = layer_to_device(lay, rank, n, k)
    bias = torch.from_numpy(s["b"]).to("cuda").to(torch.bfloat16)
    y = svdq.svdq_linear_w4a4(t_x(s["x"], True), d, bias=bias)
    y_ref, _ = O.linear_w4a4(s["x"], lay, s["b"])
    assert_y_close(y, y_ref, False, f"{m}x{k}x{n} r{rank}")


def test_linear_deterministic_and_fully_written():
    s = synth.layer(200, 1024, 336, 32, seed=4, workload="attn")
    lay = _oracle_layer(s["w"], s["x"], 32)
    d = layer_to_device(lay, 32, 336, 1024)
    x = t_x(s["x"], True)
    buf = torch.full((200 * 336 + 4096,), float("nan"), dtype=torch.float32, device="cuda")
    y1 = buf[:200 * 336].view(200, 336)
    svdq.svdq_linear_w4a4(x, d, Y=y1)
    torch.cuda.synchronize()
    assert not torch.isnan(y1).any(), "unwritten output elements"
    assert torch.isnan(buf[200 * 336:]).all(), "write past the end of Y"
    y2 = svdq.svdq_linear_w4a4(x, d)
    assert torch.equal(y1, y2), "two runs differ"


def test_bf16_output_is_rne_of_f32_output():
    """The bf16 output is the round-to-nearest-even bf16 of the fp32 output
    of the same call, bit for bit (the epilogue's conversion), also with the
    outputs scaled into the subnormal range and up to about 2^100."""
    s = synth.layer(300, 1024, 272, 32, seed=6, workload="attn")
    lay = _oracle_layer(s["w"], s["x"], 32)
    for scale in (1.0, 2.0 ** -128, 2.0 ** 100):
        d = layer_to_device(dict(lay, sW=(lay["sW"] * np.float32(scale)).astype(np.float32),
                                 lora_up=lay["lora_up"] * scale), 32, 272, 1024)
        x = t_x(s["x"], True)
        y32 = svdq.svdq_linear_w4a4(x, d, y_dtype=torch.float32)
        y16 = svdq.svdq_linear_w4a4(x, d, y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        f = y32.cpu().numpy()
        assert np.all(np.isfinite(f))
        assert np.array_equal(bf16_bits_np(y16), F.bf16_bits(f)), f"scale {scale}"


def test_act_absmax_matches():
    s = synth.layer(333, 1024, 16, 0, seed=5, workload="attn")
    a = svdq.svdq_act_absmax(t_x(s["x"], True))
    assert np.array_equal(a.cpu().numpy(), O.act_absmax(s["x"]))
    x2 = synth.layer(50, 1024, 16, 0, seed=6, workload="attn")["x"]
    a = svdq.svdq_act_absmax(t_x(x2, True), a)
    assert np.array_equal(a.cpu().numpy(), np.maximum(O.act_absmax(s["x"]), O.act_absmax(x2)))


# ------------------------------------------------------- offline quantizer

def test_quantize_weights_given_lowrank_bit_exact():
    s = synth.small()
    amax = O.act_absmax(s["x"])
    lay = O.quantize_weights(s["w"], amax, s["rank"])
    out = svdq.svdq_quantize_weights(
        t_f32(s["w"]), t_f32(amax), s["rank"], "int4",
        lowrank=(t_bf16_bits(lay["lora_down"]), t_bf16_bits(lay["lora_up"])), residual=True)
    torch.cuda.synchronize()
    assert np.array_equal(out["smooth"].cpu().numpy(), lay["smooth"]), "smooth differs"
    assert np.array_equal(out["residual"].cpu().numpy().view(np.uint32), lay["R"].view(np.uint32)), \
        "residual differs"
    assert np.array_equal(rm_int4(out["wcodes"].cpu().numpy()), lay["wcodes"]), "weight codes differ"
    assert np.array_equal(out["wscales"].cpu().numpy().T, lay["sW"]), "weight scales differ"


def test_quantize_weights_svd_quality():
    """The library's own SVD: its low-rank split is as good as LAPACK's
    (Frobenius error of the rank-r part within 1e-3 of Eckart-Young), and the
    residual / codes it returns satisfy the quantizer's properties."""
    s = synth.small()
    amax = O.act_absmax(s["x"])
    out = svdq.svdq_quantize_weights(t_f32(s["w"]), t_f32(amax), s["rank"], "int4", residual=True)
    torch.cuda.synchronize()
    lam, smooth = O.smoothing(amax, s["w"])
    wh = s["w"].astype(np.float64) * lam.astype(np.float64)[None, :]
    _, _, sv = O.truncated_svd(wh, s["rank"])
    ey = np.sum(sv[s["rank"]:] ** 2)
    down = F.bf16_to_f32(bf16_bits_np(out["lora_down"])).astype(np.float64)
    up = F.bf16_to_f32(bf16_bits_np(out["lora_up"])).astype(np.float64)
    low = lam.astype(np.float64)[None, :] * (up @ down)
    err = np.sum((wh - low) ** 2)
    ref = O.quantize_weights(s["w"], amax, s["rank"])
    err_ref = np.sum((wh - lam.astype(np.float64)[None, :] * (ref["lora_up"] @ ref["lora_down"])) ** 2)
    # bf16 rounding of the factors adds the same kind of error to both
    assert err <= err_ref * (1 + 1e-3) + 1e-3 * ey, (err, err_ref, ey)
    # residual identity and quantizer properties on the library's own output
    r = out["residual"].cpu().numpy()
    assert np.allclose(wh - low, r, rtol=0, atol=np.abs(r).max() * 2 ** -22 + 1e-30)
    q = O.unpack_int4(rm_int4(out["wcodes"].cpu().numpy())).astype(np.float64)
    sw = np.repeat(out["wscales"].cpu().numpy().T.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(r - sw * q) <= 0.5 * sw * (1 + 2 ** -22))


@pytest.mark.parametrize("n,k", [(12288, 3072), (3072, 12288)])
def test_quantize_weights_svd_quality_flux_shapes(n, k):
    """The library's SVD at the FLUX projection shapes, rank 32: the
    Frobenius error of its (bf16) rank-32 part of the smoothed weight is
    within 0.2% of the Eckart-Young optimum sum_{i>32} sigma_i^2 (LAPACK
    singular values, float64), plus the bf16 rounding of the factors
    (2^-16 of the energy of the top 32)."""
    rank = 32
    s = synth.layer(256, k, n, rank, seed=4, workload="flagship")
    amax = O.act_absmax(s["x"])
    out = svdq.svdq_quantize_weights(t_f32(s["w"]), t_f32(amax), rank, "int4")
    torch.cuda.synchronize()
    lam, _ = O.smoothing(amax, s["w"])
    lam64 = lam.astype(np.float64)
    wh = s["w"].astype(np.float64) * lam64[None, :]
    sv = np.linalg.svd(wh, compute_uv=False)
    ey = np.sum(sv[rank:] ** 2)
    top = np.sum(sv[:rank] ** 2)
    down = F.bf16_to_f32(bf16_bits_np(out["lora_down"])).astype(np.float64)
    up = F.bf16_to_f32(bf16_bits_np(out["lora_up"])).astype(np.float64)
    err = np.sum((wh - lam64[None, :] * (up @ down)) ** 2)
    assert err <= ey * (1 + 2e-3) + 2.0 ** -16 * top, (err / ey, ey, top)


# ------------------------------------------------------------ full size

def test_flagship_full_size_all_rows():
    """M 4096, K 3072, N 12288, rank 32 (the benchmark's configuration):
    activation codes / scales bit-exact and Y, LR within tolerance on every
    row (every wave and row-block position of every tile)."""
    m, k, n, rank = 4096, 3072, 12288, 32
    x = synth.layer(m, k, 16, 0, seed=0)["x"]
    lay = random_int4_layer(n, k, rank, seed=0)
    d = layer_to_device(lay, rank, n, k)
    xt = t_x(x, True)
    need = svdq.svdq_workspace_bytes(m, k, rank)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = svdq.svdq_linear_w4a4(xt, d, workspace=ws, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    codes, scales, lr = svdq.workspace_views(ws, m, k, rank)
    qx, sa = O.quantize_activations(x, lay["smooth"])
    assert np.array_equal(rm_int4(codes.cpu().numpy()), O.pack_int4(qx))
    assert np.array_equal(scales.cpu().numpy().T, sa)
    y_ref, _ = O.linear_w4a4(x, lay)
    assert_y_close(y, y_ref, True, "flagship, all rows")
    assert_lr_close(lr, x, lay["lora_down"], "flagship LR")


@pytest.mark.parametrize("m,k,n,workload", [(4608, 3072, 9216, "attn"), (4608, 3072, 3072, "attn"),
                                            (4608, 12288, 3072, "mlp"), (9216, 3072, 12288, "mlp")])
def test_dit_shapes_full_size_all_rows(m, k, n, workload):
    """The DiT projection shapes at rank 32: attention QKV and output
    projections at 4608 tokens, the MLP down-projection (K 12288), the MLP
    up-projection at batch 2 (M 9216).  Activation codes / scales bit-exact,
    Y and LR within tolerance, on every row."""
    rank = 32
    x = synth.layer(m, k, 16, 0, seed=2, workload=workload)["x"]
    lay = random_int4_layer(n, k, rank, seed=2, workload=workload)
    d = layer_to_device(lay, rank, n, k)
    ws = torch.empty(svdq.svdq_workspace_bytes(m, k, rank), dtype=torch.uint8, device="cuda")
    y = svdq.svdq_linear_w4a4(t_x(x, True), d, workspace=ws, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    codes, scales, lr = svdq.workspace_views(ws, m, k, rank)
    qx, sa = O.quantize_activations(x, lay["smooth"])
    assert np.array_equal(rm_int4(codes.cpu().numpy()), O.pack_int4(qx))
    assert np.array_equal(scales.cpu().numpy().T, sa)
    y_ref, _ = O.linear_w4a4(x, lay)
    assert_y_close(y, y_ref, True, f"{workload} M{m} K{k} N{n}, all rows")
    assert_lr_close(lr, x, lay["lora_down"], "LR")


def test_linear_graph_replay_matches_eager():
    """The layer captured into a HIP graph (the benchmark replays one): every
    replay, with eager work and synchronisations in between, gives the eager
    call's output bit for bit."""
    s = synth.layer(300, 1024, 272, 32, seed=9, workload="attn")
    lay = _oracle_layer(s["w"], s["x"], 32)
    d = layer_to_device(lay, 32, 272, 1024)
    x = t_x(s["x"], True)
    bias = torch.from_numpy(s["b"]).to("cuda").to(torch.bfloat16)
    ws = torch.empty(svdq.svdq_workspace_bytes(300, 1024, 32), dtype=torch.uint8, device="cuda")
    y_eager = svdq.svdq_linear_w4a4(x, d, bias, workspace=ws, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        svdq.svdq_linear_w4a4(x, d, bias, workspace=ws, Y=y)      # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        svdq.svdq_linear_w4a4(x, d, bias, workspace=ws, Y=y)
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep} differs from the eager call"
        svdq.svdq_linear_w4a4(x, d, bias, workspace=ws, y_dtype=torch.bfloat16)   # eager in between
        torch.cuda.synchronize()


def test_linear_graph_of_consecutive_calls():
    """Three layer calls on different X / Y buffers sharing one workspace,
    captured into one HIP graph (the benchmark replays such a graph): every
    replay gives each call's eager output bit for bit, so the calls inside the
    graph stay ordered on the workspace."""
    s = synth.layer(300, 1024, 272, 32, seed=10, workload="attn")
    lay = _oracle_layer(s["w"], s["x"], 32)
    d = layer_to_device(lay, 32, 272, 1024)
    xs = [t_x(s["x"], True)] + [
        t_x(synth.activations(300, 1024, 0, synth.WORKLOADS["attn"], 20 + i), True)
        for i in range(2)]
    bias = torch.from_numpy(s["b"]).to("cuda").to(torch.bfloat16)
    ws = torch.empty(svdq.svdq_workspace_bytes(300, 1024, 32), dtype=torch.uint8, device="cuda")
    eager = [svdq.svdq_linear_w4a4(x, d, bias, workspace=ws, y_dtype=torch.bfloat16) for x in xs]
    torch.cuda.synchronize()
    assert not torch.equal(eager[0], eager[1])
    ys = [torch.empty_like(e) for e in eager]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for x, y in zip(xs, ys):
            svdq.svdq_linear_w4a4(x, d, bias, workspace=ws, Y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, y in zip(xs, ys):
            svdq.svdq_linear_w4a4(x, d, bias, workspace=ws, Y=y)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(ys, eager)):
            assert torch.equal(y, e), f"replay {rep}, call {i} differs from the eager call"
        svdq.svdq_linear_w4a4(xs[1], d, bias, workspace=ws, y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
