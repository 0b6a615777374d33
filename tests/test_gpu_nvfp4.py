"""GPU parity of the NVFP4 precision of the SVDQuant layer against the CPU
oracle, through the C ABI: activation codes / E4M3 block scales bit-exact,
exact block sums in unit-scale mode, Y within 1e-2 rms(Y), the offline
quantizer's codes / scales / tensor scales bit-exact for a given low-rank
split, and the full MLP-up shape (M 4608, K 3072, N 12288, rank 32) on
sampled rows."""

import numpy as np
import pytest
import torch

from oracle import svdq as O
from oracle import nvfp4 as O4
from oracle import formats as F
from w4a4_quantized_diffusion_amd import svdq, synth
from tests.gpu_helpers import (t_f32, t_x, t_u8, t_bf16_bits, random_int4_layer,
                               assert_lr_close, assert_y_close, gm_codes, rm_codes,
                               degenerate_activations)

pytestmark = pytest.mark.gpu


def chunk_scales(sb):
    """Row-major E4M3 block scales [rows, K/16] -> chunk-major [K/64, rows, 4]."""
    sb = np.asarray(sb, dtype=np.uint8)
    rows, kb = sb.shape
    return np.ascontiguousarray(sb.reshape(rows, kb // 4, 4).transpose(1, 0, 2))


def rm_scales(cs):
    """Chunk-major [K/64, rows, 4] -> row-major [rows, K/16]."""
    cs = np.asarray(cs, dtype=np.uint8)
    g, rows, _ = cs.shape
    return np.ascontiguousarray(cs.transpose(1, 0, 2).reshape(rows, g * 4))


def nv_layer_to_device(lay, rank, n, k):
    d = dict(rank=rank, prec=svdq.NVFP4, N=n, K=k)
    d["smooth"] = t_f32(lay["smooth"])
    z = torch.zeros(1, dtype=torch.int16, device="cuda")
    d["lora_down"] = t_bf16_bits(lay["lora_down"]) if rank else z
    d["lora_up"] = t_bf16_bits(lay["lora_up"]) if rank else z
    d["wcodes"] = t_u8(gm_codes(O.pack_nibbles(lay["codes"])))
    d["wscales"] = t_u8(chunk_scales(lay["sbw"]))
    d["w_tensor_scale"] = t_f32(np.array([lay["ts_w"]], np.float32))
    d["x_tensor_scale"] = t_f32(np.array([lay["ts_x"]], np.float32))
    return d


def _oracle_layer(w, x, rank):
    return O4.quantize_weights(w, O.act_absmax(x), rank)


def _check_act(x_np, lay, rank, bf16):
    m, k = x_np.shape
    d = nv_layer_to_device(lay, rank, lay["codes"].shape[0], k)
    codes, scales, lr = svdq.svdq_act_quantize(t_x(x_np, bf16), d)
    torch.cuda.synchronize()
    e, sb = O4.quantize_activations(x_np, lay["smooth"], lay["ts_x"])
    assert np.array_equal(rm_codes(codes.cpu().numpy()), O.pack_nibbles(e)), "E2M1 codes differ"
    assert np.array_equal(rm_scales(scales.cpu().numpy()), sb), "E4M3 block scales differ"
    if rank:
        mism = assert_lr_close(lr, x_np, lay["lora_down"], "LR")
        assert mism <= 0.01 * lr.numel(), f"{mism} LR entries differ from the oracle's bits"


def test_nvfp4_act_quant_small_workload_fp32():
    s = synth.small()
    _check_act(s["x"], _oracle_layer(s["w"], s["x"], s["rank"]), s["rank"], bf16=False)


@pytest.mark.parametrize("m", [1, 100, 257])
def test_nvfp4_act_quant_bf16_ragged_rows(m):
    s = synth.layer(m, 3072, 256, 32, seed=11, workload="mlp_fp4")
    _check_act(s["x"], _oracle_layer(s["w"], s["x"], 32), 32, bf16=True)


@pytest.mark.parametrize("rank", [32, 48])
def test_nvfp4_act_quant_large_m(rank):
    """M 4104: 8-row 4-wave workgroups with prefetched lora_down."""
    s = synth.layer(4104, 3072, 64, rank, seed=12, workload="mlp_fp4")
    _check_act(s["x"], _oracle_layer(s["w"], s["x"], rank), rank, bf16=True)


def test_nvfp4_act_quant_grid_midpoints():
    """Block amax 12 with tensor scale 1 gives the block scale 2.0, so the
    quotients z / 2 are exact: every E2M1 midpoint (0.25 ... 5), one ulp on
    either side of it, both signs, and the ties that round to zero.  Codes
    and scales must match the oracle bit for bit."""
    k, m = 256, 16
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(9))])
    vals = np.concatenate([vals, -vals]) * np.float32(2.0)     # z = 2 t
    x = np.zeros((m, k), np.float32)
    for r in range(m):
        for b in range(k // 16):
            x[r, 16 * b] = 12.0 if (r + b) % 2 else -12.0
            for i in range(1, 16):
                x[r, 16 * b + i] = vals[(r * 7 + b * 15 + i) % vals.size]
    lay = dict(smooth=np.ones(k, np.float32), ts_x=np.float32(1.0), ts_w=np.float32(1.0),
               codes=np.zeros((16, k), np.uint8), sbw=np.zeros((16, k // 16), np.uint8),
               lora_down=None, lora_up=None)
    _check_act(x, lay, 0, bf16=False)


def test_nvfp4_act_quant_block_scale_ties():
    """Tensor scale 1 (divisor 6): block amaxes whose quotient a / 6 is an
    E4M3 grid point, a midpoint between two (normal and subnormal range), one
    ulp on either side of it, and values past 448 that saturate.  The block
    scales and the codes they lead to must match the oracle bit for bit."""
    vals = F.E4M3_POS[1:]
    mids = (vals[1:] + vals[:-1]) / 2
    a = (np.concatenate([vals, mids]) * 6).astype(np.float32)
    a = a[(a > 0) & np.isfinite(a)]
    amax = np.concatenate([a, np.nextafter(a, np.float32(0)), np.nextafter(a, np.float32(1e9)),
                           np.array([2700, 2784, 2800, 1e5], np.float32)])
    k = 256
    m = -(-amax.size // (k // 16))
    x = np.zeros((m, k), np.float32)
    g = np.random.default_rng(5)
    for i, v in enumerate(amax):
        r, b_ = divmod(i, k // 16)
        blk = g.uniform(-1, 1, 16).astype(np.float32) * v
        blk[(i * 7) % 16] = v if i % 2 else -v
        x[r, 16 * b_:16 * b_ + 16] = blk
    lay = dict(smooth=np.ones(k, np.float32), ts_x=np.float32(1.0), ts_w=np.float32(1.0),
               codes=np.zeros((16, k), np.uint8), sbw=np.zeros((16, k // 16), np.uint8),
               lora_down=None, lora_up=None)
    _check_act(x, lay, 0, bf16=False)


@pytest.mark.parametrize("ts", [1.0, 3.0e-5])
def test_nvfp4_act_quant_degenerate_inputs(ts):
    """All-zero rows and blocks, constant blocks, subnormal and huge values,
    block scales that round to zero or saturate at 448: codes and scales
    bit-exact against the oracle, for two tensor scales."""
    x = degenerate_activations(seed=4)
    k = x.shape[1]
    lay = dict(smooth=np.ones(k, np.float32), ts_x=np.float32(ts), ts_w=np.float32(1.0),
               codes=np.zeros((16, k), np.uint8), sbw=np.zeros((16, k // 16), np.uint8),
               lora_down=None, lora_up=None)
    _check_act(x, lay, 0, bf16=False)


def _random_e2m1(g, shape):
    """Random E2M1 nibbles without the negative zero 0x8 (the quantizer
    never writes it)."""
    c = g.integers(0, 15, shape).astype(np.uint8)
    return np.where(c >= 8, c + 1, c).astype(np.uint8)


def test_nvfp4_gemm_unit_scale_exact():
    """rank 0, every block scale 1 (E4M3 0x38), tensor scales 1, no bias,
    fp32 out: Y is the exact sum of E2M1 products (multiples of 1/4 far
    below 2^22, so exact in fp32).  Ragged M and N, several tiles."""
    g = np.random.default_rng(21)
    m, k, n = 300, 384, 272
    ex = _random_e2m1(g, (m, k))
    ew = _random_e2m1(g, (n, k))
    ex[0, :] = 7                                  # 6 * -6 everywhere
    ew[0, :] = 15
    one = np.full((m, k // 16), 0x38, np.uint8)
    lay = dict(rank=0, prec=svdq.NVFP4, N=n, K=k, wcodes=t_u8(gm_codes(O.pack_nibbles(ew))),
               wscales=t_u8(chunk_scales(np.full((n, k // 16), 0x38, np.uint8))),
               lora_up=None, w_tensor_scale=t_f32(np.ones(1)), x_tensor_scale=t_f32(np.ones(1)))
    y = svdq.svdq_gemm_w4a4(t_u8(gm_codes(O.pack_nibbles(ex))), t_u8(chunk_scales(one)), None,
                            lay)
    ref = F.e2m1_decode(ex) @ F.e2m1_decode(ew).T
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


def test_nvfp4_gemm_single_block_scaled():
    """Only block 5 non-zero, random E4M3 block scales (subnormal codes
    included) and power-of-two tensor scales: every output is one exact
    product sbx sbw P_5 ts_x ts_w."""
    g = np.random.default_rng(22)
    m, k, n = 96, 256, 160
    ex = np.zeros((m, k), np.uint8)
    ew = np.zeros((n, k), np.uint8)
    ex[:, 80:96] = _random_e2m1(g, (m, 16))
    ew[:, 80:96] = _random_e2m1(g, (n, 16))
    sbx = g.integers(0x01, 0x7F, (m, k // 16)).astype(np.uint8)
    sbw = g.integers(0x01, 0x7F, (n, k // 16)).astype(np.uint8)
    lay = dict(rank=0, prec=svdq.NVFP4, N=n, K=k, wcodes=t_u8(gm_codes(O.pack_nibbles(ew))),
               wscales=t_u8(chunk_scales(sbw)), lora_up=None,
               w_tensor_scale=t_f32(np.array([0.25])), x_tensor_scale=t_f32(np.array([8.0])))
    y = svdq.svdq_gemm_w4a4(t_u8(gm_codes(O.pack_nibbles(ex))), t_u8(chunk_scales(sbx)), None,
                            lay)
    p5 = F.e2m1_decode(ex[:, 80:96]) @ F.e2m1_decode(ew[:, 80:96]).T
    ref = 2.0 * F.e4m3_decode(sbx[:, 5])[:, None] * F.e4m3_decode(sbw[:, 5])[None, :] * p5
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("ybf16", [False, True])
def test_nvfp4_linear_small_workload(ybf16):
    s = synth.small()
    lay = _oracle_layer(s["w"], s["x"], s["rank"])
    d = nv_layer_to_device(lay, s["rank"], 1024, 1024)
    y = svdq.svdq_linear_w4a4(t_x(s["x"], False), d, bias=t_f32(s["b"]),
                              y_dtype=torch.bfloat16 if ybf16 else torch.float32)
    y_ref, _ = O4.linear_nvfp4(s["x"], lay, s["b"])
    assert_y_close(y, y_ref, ybf16, "NVFP4 small workload")


@pytest.mark.parametrize("m,k,n,rank", [(77, 192, 48, 16), (300, 1024, 272, 32),
                                        (129, 640, 144, 0), (5, 3072, 400, 48),
                                        (1, 64, 16, 0), (300, 64, 272, 32)])
def test_nvfp4_linear_ragged_shapes(m, k, n, rank):
    s = synth.layer(m, k, n, rank, seed=13, workload="mlp_fp4")
    lay = _oracle_layer(s["w"], s["x"], rank)
    d = nv_layer_to_device(lay, rank, n, k)
    bias = torch.from_numpy(s["b"]).to("cuda").to(torch.bfloat16)
    y = svdq.svdq_linear_w4a4(t_x(s["x"], True), d, bias=bias)
    y_ref, _ = O4.linear_nvfp4(s["x"], lay, s["b"])
    assert_y_close(y, y_ref, False, f"NVFP4 {m}x{k}x{n} r{rank}")


def test_nvfp4_quantize_weights_given_lowrank_bit_exact():
    s = synth.small()
    amax = O.act_absmax(s["x"])
    lay = O4.quantize_weights(s["w"], amax, s["rank"])
    out = svdq.svdq_quantize_weights(
        t_f32(s["w"]), t_f32(amax), s["rank"], "nvfp4",
        lowrank=(t_bf16_bits(lay["lora_down"]), t_bf16_bits(lay["lora_up"])), residual=True)
    torch.cuda.synchronize()
    assert np.array_equal(out["smooth"].cpu().numpy(), lay["smooth"]), "smooth differs"
    assert np.array_equal(out["residual"].cpu().numpy().view(np.uint32),
                          lay["R"].view(np.uint32)), "residual differs"
    assert out["w_tensor_scale"].item() == lay["ts_w"], "weight tensor scale differs"
    assert out["x_tensor_scale"].item() == lay["ts_x"], "activation tensor scale differs"
    assert np.array_equal(rm_codes(out["wcodes"].cpu().numpy()), lay["wcodes"]), "codes differ"
    assert np.array_equal(rm_scales(out["wscales"].cpu().numpy()), lay["sbw"]), "scales differ"


@pytest.mark.parametrize("m,k,n", [(4608, 3072, 12288), (4608, 12288, 3072), (9216, 3072, 12288)])
def test_nvfp4_mlp_full_size_all_rows(m, k, n):
    """The MLP pair at rank 32: up-projection (K 3072 -> N 12288) at 4608
    tokens and at batch 2 (M 9216), down-projection (K 12288 -> N 3072).
    Activation codes / scales bit-exact and Y within tolerance on every row."""
    rank = 32
    x = synth.layer(m, k, 16, 0, seed=0, workload="mlp_fp4")["x"]
    base = random_int4_layer(n, k, rank, seed=0, workload="mlp_fp4")
    g = np.random.default_rng(23)
    lay = dict(smooth=base["smooth"], lora_down=base["lora_down"], lora_up=base["lora_up"],
               codes=_random_e2m1(g, (n, k)),
               sbw=g.integers(0x20, 0x48, (n, k // 16)).astype(np.uint8),
               ts_w=np.float32(0.0123),
               ts_x=O4.tensor_scale(np.max(F.fl32(O.act_absmax(x).astype(np.float64)
                                                  * base["smooth"].astype(np.float64)))))
    d = nv_layer_to_device(lay, rank, n, k)
    need = svdq.svdq_workspace_bytes(m, k, rank, "nvfp4")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = svdq.svdq_linear_w4a4(t_x(x, True), d, workspace=ws, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    codes, scales, lr = svdq.workspace_views(ws, m, k, rank, "nvfp4")
    e, sb = O4.quantize_activations(x, lay["smooth"], lay["ts_x"])
    assert np.array_equal(rm_codes(codes.cpu().numpy()), O.pack_nibbles(e))
    assert np.array_equal(rm_scales(scales.cpu().numpy()), sb)
    y_ref, _ = O4.linear_nvfp4(x, lay)
    assert_y_close(y, y_ref, True, f"MLP M{m} K{k} N{n}, all rows")


def test_nvfp4_linear_deterministic_and_fully_written():
    """Two runs give the same bits; every element of Y is written and
    nothing past its end (Y inside a NaN-filled buffer)."""
    s = synth.layer(200, 1024, 336, 32, seed=4, workload="mlp_fp4")
    lay = _oracle_layer(s["w"], s["x"], 32)
    d = nv_layer_to_device(lay, 32, 336, 1024)
    x = t_x(s["x"], True)
    buf = torch.full((200 * 336 + 4096,), float("nan"), dtype=torch.float32, device="cuda")
    y1 = buf[:200 * 336].view(200, 336)
    svdq.svdq_linear_w4a4(x, d, Y=y1)
    torch.cuda.synchronize()
    assert not torch.isnan(y1).any(), "unwritten output elements"
    assert torch.isnan(buf[200 * 336:]).all(), "write past the end of Y"
    y2 = svdq.svdq_linear_w4a4(x, d)
    assert torch.equal(y1, y2), "two runs differ"
