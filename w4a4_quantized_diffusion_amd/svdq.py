"""Python binding of the C ABI in include/svdq.h (argument marshalling only).

Every function here has the name of the C entry point it calls.  Tensors
are torch tensors on the current HIP device (PyTorch provides device memory
and the stream); every step of the layer runs in the library's kernels.  If
the library is not built this module raises; there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")

INT4, NVFP4 = 0, 1
F32, BF16 = 0, 1
LOWRANK_GIVEN = 1

_PREC = {"int4": INT4, "nvfp4": NVFP4, INT4: INT4, NVFP4: NVFP4}
_DT = {torch.float32: F32, torch.bfloat16: BF16}

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_SIG = {
    "svdq_last_error": (ctypes.c_char_p, []),
    "svdq_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I32, ctypes.c_int]),
    "svdq_workspace_layout": (None, [_I64, _I64, _I32, ctypes.c_int, _P, _P, _P]),
    "svdq_act_absmax": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, _P]),
    "svdq_quantize_weights": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, ctypes.c_int, _U32,
                                              _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "svdq_act_quantize": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I32, ctypes.c_int,
                                          _P, _P, _P, _P, _P, _P, _P]),
    "svdq_act_quantize_gelu": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I32, ctypes.c_int,
                                               _P, _P, _P, _P, _P, _P, _P]),
    "svdq_gemm_w4a4": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I32, ctypes.c_int, _P, _P,
                                       _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int, _P]),
    # X, x_dtype, M, K, N, rank, prec, smooth, lora_down, lora_up, wcodes,
    # wscales, w_tensor_scale, x_tensor_scale, bias, bias_dtype, Y, y_dtype,
    # workspace, workspace_bytes, stream
    "svdq_linear_w4a4": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _I32, ctypes.c_int,
                                         _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _P,
                                         ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "svdq_linear_w4a4_gelu": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _I32,
                                              ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_int, _P, ctypes.c_int, _P, ctypes.c_size_t,
                                              _P]),
    "svdq_noalloc_max_workspace_bytes": (ctypes.c_size_t, []),
    "svdq_linear_w4a4_noalloc": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _I32,
                                                 ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P,
                                                 ctypes.c_int, _P, ctypes.c_int, _P]),
    "svdq_fold_lora": (ctypes.c_int, [_P, _P, _I64, _I64, _I32, _P, _P, _I32, ctypes.c_float,
                                       _P, _P, _P, _P]),
    "awq_quantize_weights": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, _P]),
    "awq_linear_w4a16": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P,
                                         ctypes.c_int, _P]),
}
EXPORTS = tuple(_SIG)


class SvdqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def lib():
    """Load libsvdq.so (built in place by the package's build step)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def svdq_last_error():
    return lib().svdq_last_error().decode()


def _check(st):
    if st != 0:
        raise SvdqError(st, svdq_last_error())


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


# ----------------------------------------------------------------- calls

def svdq_workspace_bytes(M, K, rank, prec="int4"):
    return int(lib().svdq_workspace_bytes(M, K, rank, _PREC[prec]))


def svdq_workspace_layout(M, K, rank, prec="int4"):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    lib().svdq_workspace_layout(M, K, rank, _PREC[prec], ctypes.byref(a), ctypes.byref(b),
                                ctypes.byref(c))
    return a.value, b.value, c.value


def svdq_act_absmax(X, amax=None):
    """Fold max|X[:, k]| into amax (float32 [K]); returns amax."""
    M, K = X.shape
    if amax is None:
        amax = torch.zeros(K, dtype=torch.float32, device=X.device)
    _check(lib().svdq_act_absmax(_p(X), _DT[X.dtype], M, K, _p(amax), _stream()))
    return amax


def svdq_quantize_weights(W, act_amax, rank, prec="int4", lowrank=None, residual=False):
    """Offline quantization of W [N, K] float32.  Returns a dict of device
    tensors: smooth, lora_down, lora_up, wcodes, wscales, w_tensor_scale,
    x_tensor_scale (NVFP4), residual (if asked), rank, prec."""
    N, K = W.shape
    dev = W.device
    pr = _PREC[prec]
    out = dict(rank=rank, prec=pr, N=N, K=K)
    out["smooth"] = _empty((K,), torch.float32, dev)
    flags = 0
    if lowrank is not None:
        down, up = lowrank
        out["lora_down"], out["lora_up"] = down.contiguous(), up.contiguous()
        flags = LOWRANK_GIVEN
    else:
        out["lora_down"] = _empty((rank, K), torch.int16, dev)
        out["lora_up"] = _empty((N, rank), torch.int16, dev)
    # chunk-major along K: codes [K/64][N][32]; scales [K/64][N] f32 (INT4)
    # or [K/64][N][4] E4M3 bytes (NVFP4)
    out["wcodes"] = _empty((K // 64, N, 32), torch.uint8, dev)
    if pr == INT4:
        out["wscales"] = _empty((K // 64, N), torch.float32, dev)
    else:
        out["wscales"] = _empty((K // 64, N, 4), torch.uint8, dev)
    out["w_tensor_scale"] = torch.ones(1, dtype=torch.float32, device=dev)
    out["x_tensor_scale"] = torch.ones(1, dtype=torch.float32, device=dev)
    out["residual"] = _empty((N, K), torch.float32, dev) if residual else None
    _check(lib().svdq_quantize_weights(
        _p(W), N, K, _p(act_amax), rank, pr, flags, _p(out["smooth"]),
        _p(out["lora_down"]) if rank else None, _p(out["lora_up"]) if rank else None,
        _p(out["wcodes"]), _p(out["wscales"]), _p(out["w_tensor_scale"]),
        _p(out["x_tensor_scale"]), _p(out["residual"]), _stream()))
    return out


def svdq_act_quantize(X, layer, codes=None, scales=None, LR=None, _entry="svdq_act_quantize"):
    """The activation kernel alone: returns (codes, scales, LR).  Codes are
    chunk-major [K/64][M][32]; scales [K/64][M] f32 (INT4) or [K/64][M][4]
    E4M3 bytes (NVFP4)."""
    M, K = X.shape
    rank, pr, dev = layer["rank"], layer["prec"], X.device
    if codes is None:
        codes = _empty((K // 64, M, 32), torch.uint8, dev)
    if scales is None:
        scales = (_empty((K // 64, M), torch.float32, dev) if pr == INT4
                  else _empty((K // 64, M, 4), torch.uint8, dev))
    if LR is None and rank:
        LR = _empty((M, rank), torch.int16, dev)
    _check(getattr(lib(), _entry)(
        _p(X), _DT[X.dtype], M, K, rank, pr, _p(layer["smooth"]),
        _p(layer["lora_down"]) if rank else None, _p(layer["x_tensor_scale"]),
        _p(codes), _p(scales), _p(LR) if rank else None, _stream()))
    return codes, scales, LR


def svdq_act_quantize_gelu(X, layer, codes=None, scales=None, LR=None):
    """svdq_act_quantize on bf16(GELU(X)) (X bf16): the MLP down-projection's
    activation step with the GELU fused in."""
    return svdq_act_quantize(X, layer, codes, scales, LR, _entry="svdq_act_quantize_gelu")


def svdq_gemm_w4a4(codes, scales, LR, layer, bias=None, y_dtype=torch.float32, Y=None):
    """The GEMM with its epilogue alone, on the activation kernel's outputs."""
    M = codes.shape[1]
    K, N, rank, pr = layer["K"], layer["N"], layer["rank"], layer["prec"]
    if Y is None:
        Y = _empty((M, N), y_dtype, codes.device)
    _check(lib().svdq_gemm_w4a4(
        _p(codes), _p(scales), _p(LR) if rank else None, M, K, N, rank, pr,
        _p(layer["wcodes"]), _p(layer["wscales"]), _p(layer["lora_up"]) if rank else None,
        _p(layer["w_tensor_scale"]), _p(layer["x_tensor_scale"]), _p(bias),
        _DT[bias.dtype] if bias is not None else F32, _p(Y), _DT[Y.dtype], _stream()))
    return Y


def svdq_linear_w4a4(X, layer, bias=None, y_dtype=torch.float32, workspace=None, Y=None,
                     _entry="svdq_linear_w4a4"):
    """The whole layer.  bias: float32 or bfloat16 [N] (any of the two,
    independent of X's dtype) or None.  Returns Y [M, N]."""
    M, K = X.shape
    N, rank, pr = layer["N"], layer["rank"], layer["prec"]
    if bias is not None and bias.dtype not in _DT:
        raise ValueError("bias must be float32 or bfloat16")
    if Y is None:
        Y = _empty((M, N), y_dtype, X.device)
    need = svdq_workspace_bytes(M, K, rank, pr)
    if workspace is None:
        workspace = _empty((max(need, 256),), torch.uint8, X.device)
    _check(getattr(lib(), _entry)(
        _p(X), _DT[X.dtype], M, K, N, rank, pr, _p(layer["smooth"]),
        _p(layer["lora_down"]) if rank else None, _p(layer["lora_up"]) if rank else None,
        _p(layer["wcodes"]), _p(layer["wscales"]), _p(layer["w_tensor_scale"]),
        _p(layer["x_tensor_scale"]), _p(bias), _DT[bias.dtype] if bias is not None else F32,
        _p(Y), _DT[Y.dtype], _p(workspace), workspace.numel(), _stream()))
    return Y


def svdq_noalloc_max_workspace_bytes():
    return int(lib().svdq_noalloc_max_workspace_bytes())


def svdq_linear_w4a4_noalloc(X, layer, bias=None, y_dtype=torch.float32, Y=None):
    """The whole layer with the library's fixed device scratch as workspace
    (no allocation by the library; Y is allocated here only when not given).
    Calls that overlap on one GPU race on the shared scratch."""
    M, K = X.shape
    N, rank, pr = layer["N"], layer["rank"], layer["prec"]
    if bias is not None and bias.dtype not in _DT:
        raise ValueError("bias must be float32 or bfloat16")
    if Y is None:
        Y = _empty((M, N), y_dtype, X.device)
    _check(lib().svdq_linear_w4a4_noalloc(
        _p(X), _DT[X.dtype], M, K, N, rank, pr, _p(layer["smooth"]),
        _p(layer["lora_down"]) if rank else None, _p(layer["lora_up"]) if rank else None,
        _p(layer["wcodes"]), _p(layer["wscales"]), _p(layer["w_tensor_scale"]),
        _p(layer["x_tensor_scale"]), _p(bias), _DT[bias.dtype] if bias is not None else F32,
        _p(Y), _DT[Y.dtype], _stream()))
    return Y


def svdq_linear_w4a4_gelu(X, layer, bias=None, y_dtype=torch.float32, workspace=None, Y=None):
    """The whole layer on bf16(GELU(X)) (X bf16): the MLP down-projection with
    the GELU fused into the activation pass."""
    return svdq_linear_w4a4(X, layer, bias, y_dtype, workspace, Y, _entry="svdq_linear_w4a4_gelu")


def _bf16_bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def svdq_fold_lora(layer, A, B, scale=1.0):
    """A layer dict whose low-rank branch also carries the LoRA adapter
    scale * B A (A [r_lora, K], B [N, r_lora], bf16 or their int16 bit
    patterns): rank becomes round_up(rank + r_lora, 16), lora_down / lora_up
    are new tensors, every other entry is shared with `layer`."""
    N, K, rank = layer["N"], layer["K"], layer["rank"]
    ref = layer.get("wcodes", layer.get("lora_down"))
    for name, t in (("A", A), ("B", B)):
        if t.dtype not in (torch.bfloat16, torch.int16):
            raise TypeError(f"{name} must be bfloat16 (or its int16 bit patterns), got {t.dtype}")
        if ref is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the layer on {ref.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    A, B = _bf16_bits(A), _bf16_bits(B)
    r_lora = A.shape[0]
    if A.dim() != 2 or A.shape[1] != K or B.dim() != 2 or tuple(B.shape) != (N, r_lora):
        raise ValueError("A must be [r_lora, K] and B [N, r_lora]")
    r_new = (rank + r_lora + 15) // 16 * 16
    dev = A.device
    down = _empty((r_new, K), torch.int16, dev)
    up = _empty((N, r_new), torch.int16, dev)
    got = ctypes.c_int32()
    _check(lib().svdq_fold_lora(
        _p(layer["lora_down"]) if rank else None, _p(layer["lora_up"]) if rank else None,
        N, K, rank, _p(A), _p(B), r_lora, float(scale), _p(down), _p(up),
        ctypes.byref(got), _stream()))
    assert got.value == r_new
    out = dict(layer)
    out.update(rank=r_new, lora_down=down, lora_up=up)
    return out


def workspace_views(workspace, M, K, rank, prec="int4"):
    """(codes, scales, LR) views of a workspace filled by svdq_linear_w4a4."""
    pr = _PREC[prec]
    c, s, l = svdq_workspace_layout(M, K, rank, pr)
    codes = workspace[c:c + M * (K // 2)].view(K // 64, M, 32)
    if pr == INT4:
        scales = workspace[s:s + M * (K // 64) * 4].view(torch.float32).view(K // 64, M)
    else:
        scales = workspace[s:s + M * (K // 16)].view(K // 64, M, 4)
    lr = workspace[l:l + M * rank * 2].view(torch.int16).view(M, rank) if rank else None
    return codes, scales, lr


def awq_quantize_weights(W, group=64):
    N, K = W.shape
    dev = W.device
    # chunk-major along K: q [K/64][N][32], scales / zeros [K/64][N]
    q = _empty((K // group, N, 32), torch.uint8, dev)
    s = _empty((K // group, N), torch.int16, dev)
    z = _empty((K // group, N), torch.int16, dev)
    _check(lib().awq_quantize_weights(_p(W), N, K, group, _p(q), _p(s), _p(z), _stream()))
    return dict(q=q, scales=s, zeros=z, N=N, K=K, group=group)


def awq_linear_w4a16(X, layer, bias=None, y_dtype=torch.bfloat16, Y=None):
    """X bf16 [M, K]; bias bf16 [N] or None."""
    M, K = X.shape
    N = layer["N"]
    if Y is None:
        Y = _empty((M, N), y_dtype, X.device)
    _check(lib().awq_linear_w4a16(
        _p(X), M, K, N, layer["group"], _p(layer["q"]), _p(layer["scales"]),
        _p(layer["zeros"]), _p(bias), _p(Y), _DT[Y.dtype], _stream()))
    return Y
