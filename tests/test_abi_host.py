"""Host-side checks of the C-ABI library (no GPU work): it loads, exports every
entry point the header declares, and rejects bad arguments with the
documented status before any HIP call."""

import ctypes
import os
import re

import pytest

from w4a4_quantized_diffusion_amd import svdq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

INVALID, UNSUPPORTED = 1, 2


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:svdq|awq)_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(svdq.LIB_PATH):
        pytest.fail("libsvdq.so is not built (run __graft_entry__.build())")
    return svdq.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("svdq_quantize_weights", "svdq_linear_w4a4", "awq_linear_w4a16",
              "svdq_act_quantize", "svdq_gemm_w4a4", "awq_quantize_weights"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(svdq.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(_declared()) == set(svdq.EXPORTS)


def test_workspace_size_and_layout(lib):
    M, K, r = 4096, 3072, 32
    n = svdq.svdq_workspace_bytes(M, K, r, "int4")
    c, s, l = svdq.svdq_workspace_layout(M, K, r, "int4")
    assert c == 0 and s >= M * K // 2 and l >= s + M * (K // 64) * 4
    assert n >= l + M * r * 2 and n % 256 == 0 and s % 256 == 0 and l % 256 == 0
    assert svdq.svdq_workspace_bytes(M, 100, r, "int4") == 0
    assert svdq.svdq_workspace_bytes(M, K, 17, "int4") == 0
    nf = svdq.svdq_workspace_bytes(M, K, r, "nvfp4")
    assert nf >= M * K // 2 + M * K // 16 + M * r * 2


@pytest.mark.parametrize("K,rank,msg", [(100, 32, "K must"), (0, 32, "K must"),
                                        (128, 17, "rank"), (128, -16, "rank"),
                                        (128, 272, "rank")])
def test_act_quantize_rejects_bad_shapes(lib, K, rank, msg):
    st = lib.svdq_act_quantize(None, 1, 64, K, rank, 0, None, None, None, None, None, None, None)
    assert st == INVALID
    assert msg in svdq.svdq_last_error()


def test_null_pointers_rejected(lib):
    st = lib.svdq_act_quantize(None, 1, 64, 128, 16, 0, None, None, None, None, None, None, None)
    assert st == INVALID and "X is NULL" in svdq.svdq_last_error()


def test_misaligned_pointer_rejected(lib):
    st = lib.svdq_act_quantize(ctypes.c_void_p(0x1002), 1, 64, 128, 0, 0, ctypes.c_void_p(0x2000),
                               None, None, ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000),
                               None, None)
    assert st == INVALID and "aligned" in svdq.svdq_last_error()


def test_unknown_enums_rejected(lib):
    assert lib.svdq_act_quantize(None, 7, 64, 128, 16, 0, None, None, None, None, None, None,
                                 None) == INVALID
    assert lib.svdq_act_quantize(None, 1, 64, 128, 16, 5, None, None, None, None, None, None,
                                 None) == INVALID


def test_gemm_rejects_bad_n(lib):
    st = lib.svdq_gemm_w4a4(None, None, None, 64, 128, 100, 16, 0, None, None, None, None, None,
                            None, 0, None, 0, None)
    assert st == INVALID and "N must" in svdq.svdq_last_error()


def test_linear_rejects_small_workspace(lib):
    p = ctypes.c_void_p
    st = lib.svdq_linear_w4a4(p(0x10000), 1, 64, 128, 64, 16, 0, p(0x20000), p(0x30000),
                              p(0x40000), p(0x50000), p(0x60000), None, None, None, 0,
                              p(0x70000), 0, p(0x100000), 100, None)
    assert st == INVALID and "workspace too small" in svdq.svdq_last_error()


def test_linear_rejects_overlap(lib):
    p = ctypes.c_void_p
    need = svdq.svdq_workspace_bytes(64, 128, 16, "int4")
    st = lib.svdq_linear_w4a4(p(0x100000), 1, 64, 128, 64, 16, 0, p(0x20000), p(0x30000),
                              p(0x40000), p(0x50000), p(0x60000), None, None, None, 0,
                              p(0x900000), 0, p(0x100000), need, None)
    assert st == INVALID and "overlap" in svdq.svdq_last_error()


def test_quantize_weights_rejects_rank(lib):
    st = lib.svdq_quantize_weights(ctypes.c_void_p(0x1000), 32, 64, None, 48, 0, 0,
                                   *([None] * 9))
    assert st == INVALID and "rank" in svdq.svdq_last_error()


def test_quantize_weights_rejects_flags(lib):
    st = lib.svdq_quantize_weights(ctypes.c_void_p(0x1000), 32, 64, None, 16, 0, 8,
                                   *([None] * 9))
    assert st == INVALID and "flags" in svdq.svdq_last_error()


def test_awq_rejects_group(lib):
    assert lib.awq_linear_w4a16(None, 1, 128, 64, 128, None, None, None, None, None, 1,
                                None) == UNSUPPORTED
    assert lib.awq_quantize_weights(None, 64, 128, 32, None, None, None, None) == UNSUPPORTED


def test_zero_rows_is_a_noop(lib):
    # M == 0: valid, nothing launched, no pointer needed
    assert lib.svdq_act_quantize(None, 1, 0, 128, 16, 0, None, None, None, None, None, None,
                                 None) == 0
    assert lib.awq_linear_w4a16(None, 0, 128, 64, 64, None, None, None, None, None, 1,
                                None) == 0


def test_smoke_inputs_are_contiguous():
    """Every tensor smoke() hands the binding is contiguous (the binding
    rejects strided tensors)."""
    import __graft_entry__ as ge
    _, _, _, layer = ge.smoke_inputs("cpu")
    for k, v in layer.items():
        if hasattr(v, "is_contiguous"):
            assert v.is_contiguous(), k


def test_gelu_forms_take_bf16_only(lib):
    # x_dtype 0 is f32: the GELU input form rejects it before touching anything
    st = lib.svdq_act_quantize_gelu(None, 0, 64, 128, 16, 0, None, None, None, None, None, None,
                                    None)
    assert st == UNSUPPORTED and "bf16" in svdq.svdq_last_error()
    st = lib.svdq_linear_w4a4_gelu(None, 0, 64, 128, 64, 16, 0, None, None, None, None, None,
                                   None, None, None, 0, None, 1, None, 0, None)
    assert st == UNSUPPORTED and "bf16" in svdq.svdq_last_error()
    # bf16 with bad shapes / NULL pointers: the usual validation
    st = lib.svdq_act_quantize_gelu(None, 1, 64, 100, 16, 0, None, None, None, None, None, None,
                                    None)
    assert st == INVALID and "K must" in svdq.svdq_last_error()
    assert lib.svdq_act_quantize_gelu(None, 1, 0, 128, 16, 0, None, None, None, None, None, None,
                                      None) == 0


def test_fold_lora_validation(lib):
    p = ctypes.c_void_p
    r = ctypes.c_int32(-1)
    f = lib.svdq_fold_lora
    # rank not a multiple of 16, rank + r_lora past 256, r_lora 0, K not a multiple of 64
    assert f(p(0x1000), p(0x2000), 64, 128, 8, p(0x3000), p(0x4000), 4, 1.0, p(0x10000),
             p(0x20000), ctypes.byref(r), None) == INVALID
    assert "rank" in svdq.svdq_last_error()
    assert f(p(0x1000), p(0x2000), 64, 128, 240, p(0x3000), p(0x4000), 17, 1.0, p(0x10000),
             p(0x20000), ctypes.byref(r), None) == INVALID
    assert "256" in svdq.svdq_last_error()
    assert f(None, None, 64, 128, 0, p(0x3000), p(0x4000), 0, 1.0, p(0x10000), p(0x20000),
             ctypes.byref(r), None) == INVALID
    assert f(None, None, 64, 100, 0, p(0x3000), p(0x4000), 4, 1.0, p(0x10000), p(0x20000),
             ctypes.byref(r), None) == INVALID
    assert f(None, None, 64, 128, 0, p(0x3000), p(0x4000), 4, float("nan"), p(0x10000),
             p(0x20000), ctypes.byref(r), None) == INVALID
    assert "finite" in svdq.svdq_last_error()
    # NULL adapter, NULL rank_out, and outputs overlapping an input
    assert f(None, None, 64, 128, 0, None, p(0x4000), 4, 1.0, p(0x10000), p(0x20000),
             ctypes.byref(r), None) == INVALID
    assert "NULL" in svdq.svdq_last_error()
    assert f(None, None, 64, 128, 0, p(0x3000), p(0x4000), 4, 1.0, p(0x10000), p(0x20000),
             None, None) == INVALID
    # A [4, 128] bf16 = 1 KiB at 0x3000 overlaps lora_down_out at 0x3200
    assert f(None, None, 64, 128, 0, p(0x3000), p(0x40000), 4, 1.0, p(0x3200), p(0x80000),
             ctypes.byref(r), None) == INVALID
    assert "overlap" in svdq.svdq_last_error()
    assert r.value == -1


def test_noalloc_rejects_workspace_beyond_the_scratch(lib):
    """The entry point that allocates nothing checks the workspace size against
    its fixed scratch before any HIP call (fake pointers are never touched)."""
    p = ctypes.c_void_p
    cap = lib.svdq_noalloc_max_workspace_bytes()
    assert cap == 32 << 20
    # INT4, K 12288, rank 32: 4608 rows fit, 9216 do not
    assert svdq.svdq_workspace_bytes(4608, 12288, 32, "int4") <= cap
    assert svdq.svdq_workspace_bytes(9216, 12288, 32, "int4") > cap
    st = lib.svdq_linear_w4a4_noalloc(p(0x10000), 1, 9216, 12288, 64, 32, 0, p(0x20000),
                                      p(0x30000), p(0x40000), p(0x50000), p(0x60000), None,
                                      None, None, 0, p(0x70000), 1, None)
    assert st == INVALID and "scratch" in svdq.svdq_last_error()
    # M == 0 launches nothing and needs no device
    assert lib.svdq_linear_w4a4_noalloc(None, 1, 0, 128, 64, 16, 0, *([None] * 8), 0, None, 1,
                                        None) == 0


def test_gemm_calls_reject_too_many_output_tiles(lib):
    """M x N beyond 2^31 - 1 tiles of 256 x 256 (the GEMMs index tiles with
    32-bit integers) is rejected before any HIP call (fake pointers are never
    touched); the largest legal M and N alone pass the size checks."""
    p = ctypes.c_void_p
    big, bign = (1 << 27) - 1, (1 << 27) - 16          # N a multiple of 16
    st = lib.svdq_gemm_w4a4(p(0x10000), p(0x20000), None, big, 64, bign, 0, 0, p(0x30000),
                            p(0x40000), None, None, None, None, 0, p(0x50000), 1, None)
    assert st == INVALID and "tiles" in svdq.svdq_last_error()
    st = lib.svdq_linear_w4a4(p(0x10000), 1, big, 64, bign, 0, 0, p(0x20000), None, None,
                              p(0x40000), p(0x50000), None, None, None, 0, p(0x70000), 1,
                              p(0x100000), 1 << 40, None)
    assert st == INVALID and "tiles" in svdq.svdq_last_error()
    st = lib.awq_linear_w4a16(p(0x10000), big, 64, bign, 64, p(0x20000), p(0x30000),
                              p(0x40000), None, p(0x50000), 1, None)
    assert st == INVALID and "tiles" in svdq.svdq_last_error()
    # 2^27 rows or columns: out of range
    st = lib.svdq_gemm_w4a4(p(0x10000), p(0x20000), None, big + 1, 64, 64, 0, 0, p(0x30000),
                            p(0x40000), None, None, None, None, 0, p(0x50000), 1, None)
    assert st == INVALID


def test_fold_lora_binding_rejects_wrong_dtype_and_device():
    """The binding checks the adapter before calling the library: an fp32 or
    fp16 adapter (whose bytes the kernel would read as bf16 bit patterns) and
    an adapter on another device than the layer are rejected."""
    import torch
    layer = {"N": 32, "K": 64, "rank": 0, "wcodes": torch.zeros(1, 32, 32, dtype=torch.uint8)}
    a = torch.zeros(4, 64, dtype=torch.bfloat16)
    b = torch.zeros(32, 4, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        svdq.svdq_fold_lora(layer, a.float(), b)
    with pytest.raises(TypeError):
        svdq.svdq_fold_lora(layer, a, b.half())
    layer_meta = dict(layer, wcodes=torch.zeros(1, 32, 32, dtype=torch.uint8, device="meta"))
    with pytest.raises(ValueError):
        svdq.svdq_fold_lora(layer_meta, a, b)
