"""Runtime nn.Linear replacement over the C ABI: the patching shim and the
quantized-layer file format.

The lite integration does not ship model-specific fused kernels: it swaps
the nn.Linear modules of an ordinary model for runtime SVDQ (W4A4) or AWQ
(W4A16) layers (chaosnode.de page, "Nunchaku Lite vs. Original";
aiphreaks.com page, "Bringing Nunchaku 4-bit Diffusion Inference to
Diffusers", Technical Breakdown and Performance Metrics).  Here:

  SVDQLinear      one quantized layer held as device tensors; forward runs
                  svdq_linear_w4a4 (or its GELU-input form) on the current
                  stream.
  AWQLinear       one AWQ W4A16 layer; forward runs awq_linear_w4a16.
  calibrate       per-input-channel max|x| of every nn.Linear's inputs
                  (svdq_act_absmax), for the smoothing step.
  quantize_linears  swaps every eligible nn.Linear of a module in place.
  save_quantized / load_quantized
                  the quantized layers of a module in one safetensors file:
                  tensors "<module name>.<field>" and a JSON header entry
                  "svdq" = {"format", "version", "layers": {name: {...}}}.

This module is marshalling only: every step of a layer runs in the HIP
library, and without it the calls raise.
"""

import json

import torch
from torch import nn

from . import svdq

FORMAT = "svdq-w4a4-layers"
# version 2: INT4 codes in the fold format (include/svdq.h), written by
# the library's quantizer; version-1 files held textbook nibbles
VERSION = 2

_SVDQ_FIELDS = ("smooth", "lora_down", "lora_up", "wcodes", "wscales", "w_tensor_scale",
                "x_tensor_scale")
_AWQ_FIELDS = ("q", "scales", "zeros")
_PREC_NAME = {svdq.INT4: "int4", svdq.NVFP4: "nvfp4"}


def _shapes_svdq(n, k, rank, prec):
    """The field shapes and dtypes of one SVDQ layer."""
    ws = ((k // 64, n), torch.float32) if prec == svdq.INT4 else ((k // 64, n, 4), torch.uint8)
    r = max(rank, 1)
    return {"smooth": ((k,), torch.float32), "lora_down": ((r, k) if rank else (1,), torch.int16),
            "lora_up": ((n, r) if rank else (1,), torch.int16),
            "wcodes": ((k // 64, n, 32), torch.uint8), "wscales": ws,
            "w_tensor_scale": ((1,), torch.float32), "x_tensor_scale": ((1,), torch.float32)}


def _shapes_awq(n, k, group):
    return {"q": ((k // group, n, 32), torch.uint8), "scales": ((k // group, n), torch.int16),
            "zeros": ((k // group, n), torch.int16)}


class _BiasCache:
    """The bias in bf16 (awq_linear_w4a16 reads a bf16 bias)."""

    def __init__(self):
        self.key, self.value = None, None

    def get(self, bias, dtype):
        if bias is None:
            return None
        key = (bias.data_ptr(), bias._version, dtype)
        if self.key != key:
            self.key, self.value = key, bias.to(dtype).contiguous()
        return self.value


class SVDQLinear(nn.Module):
    """An SVDQuant W4A4 layer in place of nn.Linear(K, N).

    `layer` is a dict as returned by svdq.svdq_quantize_weights or
    svdq.svdq_fold_lora (device tensors plus rank, prec, N, K).  The bias is
    kept in fp32 and added in fp32 by the library.  With gelu_input the
    layer computes Linear(GELU(x)) (tanh GELU fused into the activation pass;
    x must be bf16).  Inputs of any leading shape [..., K] in fp32 or bf16;
    the output has x's dtype.  The workspace is kept between calls and
    reused on the calling stream: one module must not run on two streams at
    once."""

    def __init__(self, layer, bias=None, gelu_input=False):
        super().__init__()
        self.in_features, self.out_features = int(layer["K"]), int(layer["N"])
        self.rank, self.prec = int(layer["rank"]), int(svdq._PREC[layer["prec"]])
        self.gelu_input = bool(gelu_input)
        shapes = _shapes_svdq(self.out_features, self.in_features, self.rank, self.prec)
        for f in _SVDQ_FIELDS:
            t = layer[f]
            if self.rank == 0 and f in ("lora_down", "lora_up"):
                t = torch.zeros(1, dtype=torch.int16, device=layer["smooth"].device)
            shape, dt = shapes[f]
            if tuple(t.shape) != shape or t.dtype != dt:
                raise ValueError(f"{f}: expected {shape} {dt}, got {tuple(t.shape)} {t.dtype}")
            self.register_buffer(f, t)
        if bias is not None:
            bias = bias.detach().to(torch.float32).reshape(self.out_features).contiguous()
        self.register_buffer("bias", bias)
        self._ws = None

    @classmethod
    def from_linear(cls, linear, act_amax=None, rank=32, prec="int4", gelu_input=False):
        """Quantize an nn.Linear on its (HIP) device with the library's
        offline quantizer; act_amax is its inputs' per-channel max|x| (None:
        no smoothing)."""
        w = linear.weight.detach().to(torch.float32).contiguous()
        lay = svdq.svdq_quantize_weights(w, act_amax, rank, prec)
        return cls(lay, linear.bias, gelu_input)

    def layer(self):
        d = {f: getattr(self, f) for f in _SVDQ_FIELDS}
        d.update(rank=self.rank, prec=self.prec, N=self.out_features, K=self.in_features)
        return d

    def fold_lora(self, A, B, scale=1.0):
        """Carry a LoRA adapter scale * B A in the low-rank branch from now on
        (svdq_fold_lora)."""
        lay = svdq.svdq_fold_lora(self.layer(), A, B, scale)
        self.rank = int(lay["rank"])
        self.lora_down, self.lora_up = lay["lora_down"], lay["lora_up"]
        self._ws = None

    def forward(self, x):
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected [..., {self.in_features}] input, got {tuple(x.shape)}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        m = x2.shape[0]
        need = max(svdq.svdq_workspace_bytes(m, self.in_features, self.rank, self.prec), 256)
        if self._ws is None or self._ws.numel() < need or self._ws.device != x2.device:
            self._ws = torch.empty(need, dtype=torch.uint8, device=x2.device)
        fn = svdq.svdq_linear_w4a4_gelu if self.gelu_input else svdq.svdq_linear_w4a4
        y = fn(x2, self.layer(), self.bias, y_dtype=x2.dtype, workspace=self._ws)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self):
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"rank={self.rank}, prec={_PREC_NAME[self.prec]}, bias={self.bias is not None}, "
                f"gelu_input={self.gelu_input}")


class AWQLinear(nn.Module):
    """An AWQ W4A16 layer (asymmetric INT4 weights in groups of 64, bf16
    activations) in place of nn.Linear(K, N).  Inputs bf16 [..., K]; output
    bf16."""

    def __init__(self, layer, bias=None):
        super().__init__()
        self.in_features, self.out_features = int(layer["K"]), int(layer["N"])
        self.group = int(layer["group"])
        shapes = _shapes_awq(self.out_features, self.in_features, self.group)
        for f in _AWQ_FIELDS:
            t = layer[f]
            shape, dt = shapes[f]
            if tuple(t.shape) != shape or t.dtype != dt:
                raise ValueError(f"{f}: expected {shape} {dt}, got {tuple(t.shape)} {t.dtype}")
            self.register_buffer(f, t)
        if bias is not None:
            bias = bias.detach().to(torch.float32).reshape(self.out_features).contiguous()
        self.register_buffer("bias", bias)
        self._bias = _BiasCache()

    @classmethod
    def from_linear(cls, linear, group=64):
        lay = svdq.awq_quantize_weights(linear.weight.detach().to(torch.float32).contiguous(), group)
        return cls(lay, linear.bias)

    def forward(self, x):
        if x.dtype != torch.bfloat16:
            raise TypeError("AWQLinear takes bf16 activations")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected [..., {self.in_features}] input, got {tuple(x.shape)}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        lay = dict(q=self.q, scales=self.scales, zeros=self.zeros, N=self.out_features,
                   K=self.in_features, group=self.group)
        y = svdq.awq_linear_w4a16(x2, lay, self._bias.get(self.bias, torch.bfloat16))
        return y.reshape(*lead, self.out_features)

    def extra_repr(self):
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"group={self.group}, bias={self.bias is not None}")


# ------------------------------------------------------------ patching shim

def eligible(linear, rank=0):
    """Whether the kernels take this nn.Linear: K a multiple of 64, N of 16,
    rank at most min(N, K)."""
    return (isinstance(linear, nn.Linear) and linear.in_features % 64 == 0
            and linear.out_features % 16 == 0 and rank <= min(linear.in_features,
                                                              linear.out_features))


def calibrate(module, run):
    """Per-input-channel max|x| of the inputs of every nn.Linear in `module`
    while `run()` executes (fp32 or bf16 inputs).  Returns {name: amax}."""
    amax, hooks = {}, []

    def hook(name):
        def f(mod, args):
            x = args[0]
            x2 = x.reshape(-1, x.shape[-1]).contiguous()
            if name not in amax:
                amax[name] = torch.zeros(x2.shape[-1], dtype=torch.float32, device=x2.device)
            svdq.svdq_act_absmax(x2, amax[name])
        return f

    for name, mod in module.named_modules():
        if isinstance(mod, nn.Linear):
            hooks.append(mod.register_forward_pre_hook(hook(name)))
    try:
        with torch.no_grad():
            run()
    finally:
        for h in hooks:
            h.remove()
    return amax


def _set_child(root, name, new):
    parent = root
    parts = name.split(".")
    for p in parts[:-1]:
        parent = getattr(parent, p)
    setattr(parent, parts[-1], new)


def quantize_linears(module, act_amax=None, rank=32, prec="int4", awq=(), gelu_input=(),
                     skip=()):
    """Swap the nn.Linear modules of `module` in place: names in `awq` become
    AWQLinear, names in `skip` stay, the other eligible ones become
    SVDQLinear (gelu_input for names in `gelu_input`).  act_amax: {name:
    amax} from calibrate (a missing name quantizes without smoothing).
    Returns {name: kind}."""
    if rank < 0 or rank > 256 or rank % 16:
        raise ValueError("rank must be a multiple of 16 in [0, 256]")
    act_amax = act_amax or {}
    done = {}
    targets = [(n, m) for n, m in module.named_modules() if isinstance(m, nn.Linear)]
    for name, lin in targets:
        if name in skip:
            continue
        if name in awq:
            if not eligible(lin):
                raise ValueError(f"{name}: shape {lin.out_features}x{lin.in_features} not supported")
            _set_child(module, name, AWQLinear.from_linear(lin))
            done[name] = "awq"
        elif eligible(lin, rank):
            _set_child(module, name, SVDQLinear.from_linear(lin, act_amax.get(name), rank, prec,
                                                            name in gelu_input))
            done[name] = "svdq"
    return done


# ------------------------------------------------------------- file format

def save_quantized(module, path):
    """Write every SVDQLinear / AWQLinear of `module` to a safetensors file."""
    from safetensors.torch import save_file
    tensors, layers = {}, {}
    for name, mod in module.named_modules():
        if isinstance(mod, SVDQLinear):
            layers[name] = {"kind": "svdq", "prec": _PREC_NAME[mod.prec], "rank": mod.rank,
                            "N": mod.out_features, "K": mod.in_features,
                            "gelu_input": mod.gelu_input, "bias": mod.bias is not None}
            fields = _SVDQ_FIELDS
        elif isinstance(mod, AWQLinear):
            layers[name] = {"kind": "awq", "group": mod.group, "N": mod.out_features,
                            "K": mod.in_features, "bias": mod.bias is not None}
            fields = _AWQ_FIELDS
        else:
            continue
        for f in fields + (("bias",) if mod.bias is not None else ()):
            tensors[f"{name}.{f}"] = getattr(mod, f).detach().cpu().contiguous()
    meta = {"format": FORMAT, "version": VERSION, "layers": layers}
    save_file(tensors, path, metadata={"svdq": json.dumps(meta)})
    return list(layers)


def load_quantized(module, path, device=None):
    """Put the layers stored by save_quantized into `module` (usually the
    unquantized model's skeleton), replacing the modules of the same names.
    Every tensor is checked against the shapes its header entry implies."""
    from safetensors import safe_open
    with safe_open(path, framework="pt", device="cpu") as f:
        raw = (f.metadata() or {}).get("svdq")
        if raw is None:
            raise ValueError(f"{path}: no svdq header entry")
        meta = json.loads(raw)
        if meta.get("format") != FORMAT or meta.get("version") != VERSION:
            raise ValueError(f"{path}: format {meta.get('format')} v{meta.get('version')} "
                             f"is not {FORMAT} v{VERSION}")
        keys = set(f.keys())

        def take(name, field):
            k = f"{name}.{field}"
            if k not in keys:
                raise ValueError(f"{path}: missing tensor {k}")
            t = f.get_tensor(k)
            return t.to(device) if device is not None else t

        for name, d in meta["layers"].items():
            n, k = int(d["N"]), int(d["K"])
            bias = take(name, "bias") if d.get("bias") else None
            if d["kind"] == "svdq":
                lay = {fld: take(name, fld) for fld in _SVDQ_FIELDS}
                lay.update(rank=int(d["rank"]), prec=svdq._PREC[d["prec"]], N=n, K=k)
                new = SVDQLinear(lay, bias, bool(d.get("gelu_input", False)))
            elif d["kind"] == "awq":
                lay = {fld: take(name, fld) for fld in _AWQ_FIELDS}
                lay.update(N=n, K=k, group=int(d["group"]))
                new = AWQLinear(lay, bias)
            else:
                raise ValueError(f"{path}: unknown layer kind {d['kind']!r}")
            if bias is not None and tuple(bias.shape) != (n,):
                raise ValueError(f"{name}.bias: expected ({n},)")
            _set_child(module, name, new)
    return list(meta["layers"])
