"""GPU checks of the nn.Linear shim over the C ABI: SVDQLinear / AWQLinear
give exactly what the C entry points give, the INT4 layer matches the oracle
on its own quantized tensors, a patched block (calibrated, with the GELU
fused into the down-projection) follows the float block, and a saved and
reloaded model reproduces its outputs bit for bit."""

import numpy as np
import pytest
import torch
from torch import nn

from oracle import svdq as O
from oracle import formats as F
from w4a4_quantized_diffusion_amd import linear as L
from w4a4_quantized_diffusion_amd import svdq, synth
from tests.gpu_helpers import rm_int4, bf16_bits_np, assert_y_close

pytestmark = pytest.mark.gpu


def _linear(k, n, seed, bias=True):
    torch.manual_seed(seed)
    lin = nn.Linear(k, n, bias=bias)
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(synth.gaussian((n, k), 0.02, seed, synth.WORKLOADS["attn"], 1)))
        if bias:
            lin.bias.copy_(torch.from_numpy(synth.gaussian((n,), 0.02, seed, synth.WORKLOADS["attn"], 2)))
    return lin.cuda()


def _x(m, k, seed):
    return torch.from_numpy(synth.activations(m, k, seed, synth.WORKLOADS["attn"], 0)).cuda().to(torch.bfloat16)


def _oracle_layer(mod):
    """The device layer of an INT4 SVDQLinear in the oracle's dict form."""
    d = dict(smooth=mod.smooth.cpu().numpy(),
             q=O.unpack_int4(rm_int4(mod.wcodes.cpu().numpy())),
             sW=np.ascontiguousarray(mod.wscales.cpu().numpy().T))
    if mod.rank:
        d["lora_down"] = F.bf16_to_f32(bf16_bits_np(mod.lora_down)).astype(np.float64)
        d["lora_up"] = F.bf16_to_f32(bf16_bits_np(mod.lora_up)).astype(np.float64)
    else:
        d["lora_down"] = np.zeros((0, mod.in_features))
        d["lora_up"] = np.zeros((mod.out_features, 0))
    return d


def test_svdq_linear_matches_abi_and_oracle():
    print("SVDQLinear 2x150x512 -> 272 rank 32", flush=True)
    lin = _linear(512, 272, 0)
    x = _x(300, 512, 1).reshape(2, 150, 512)
    amax = svdq.svdq_act_absmax(x.reshape(-1, 512))
    mod = L.SVDQLinear.from_linear(lin, amax, rank=32)
    y = mod(x)
    assert y.shape == (2, 150, 272) and y.dtype == torch.bfloat16
    ws = torch.empty(svdq.svdq_workspace_bytes(300, 512, 32), dtype=torch.uint8, device="cuda")
    # the module adds its fp32 bias through the C entry point's bias_dtype
    y_abi = svdq.svdq_linear_w4a4(x.reshape(300, 512), mod.layer(), lin.bias.detach().float(),
                                  y_dtype=torch.bfloat16, workspace=ws)
    assert torch.equal(y.reshape(300, 272), y_abi)
    xb = x.reshape(300, 512).float().cpu().numpy()
    bias = lin.bias.detach().cpu().numpy().astype(np.float64)
    y_ref, _ = O.linear_w4a4(xb, _oracle_layer(mod), bias)
    assert_y_close(y.reshape(300, 272), y_ref, True, "SVDQLinear")
    # fp32 input, fp32 output, same layer
    y32 = mod(x.float())
    assert y32.dtype == torch.float32
    assert_y_close(y32.reshape(300, 272), y_ref, False, "SVDQLinear fp32")


def test_awq_linear_matches_abi():
    print("AWQLinear 7x512 -> 256", flush=True)
    lin = _linear(512, 256, 2)
    mod = L.AWQLinear.from_linear(lin)
    x = _x(7, 512, 3)
    y = mod(x)
    lay = dict(q=mod.q, scales=mod.scales, zeros=mod.zeros, N=256, K=512, group=64)
    assert torch.equal(y, svdq.awq_linear_w4a16(x, lay, lin.bias.detach().to(torch.bfloat16)))
    ref = x.float() @ lin.weight.detach().T + lin.bias.detach()
    assert (y.float() - ref).norm() / ref.norm() < 0.1


class MLP(nn.Module):
    def __init__(self, d, h):
        super().__init__()
        self.up = nn.Linear(d, h)
        self.act = nn.GELU(approximate="tanh")
        self.down = nn.Linear(h, d)
        self.gate = nn.Linear(d, d)

    def forward(self, x):
        return self.down(self.act(self.up(x))) + self.gate(x)


def _mlp(seed):
    torch.manual_seed(seed)
    m = MLP(256, 1024)
    with torch.no_grad():
        for lin in (m.up, m.down, m.gate):
            lin.weight.mul_(0.5)
    return m.cuda()


@pytest.mark.parametrize("prec", ["int4", "nvfp4"])
def test_patched_block_follows_float_and_reloads(tmp_path, prec):
    print(f"patched MLP 2x96x256 (up / GELU-fused down / AWQ gate), {prec}", flush=True)
    model = _mlp(4)
    x = _x(192, 256, 5).reshape(2, 96, 256)
    with torch.no_grad():
        y_float = model(x.float())
    amax = L.calibrate(model, lambda: model(x.float()))
    assert set(amax) == {"up", "down", "gate"}
    done = L.quantize_linears(model, amax, rank=32, prec=prec, awq={"gate"}, gelu_input={"down"})
    assert done == {"up": "svdq", "down": "svdq", "gate": "awq"}
    model.act = nn.Identity()                       # the GELU now runs inside `down`
    with torch.no_grad():
        y = model(x)
    err = ((y.float() - y_float).norm() / y_float.norm()).item()
    assert err < 0.08, err
    # the same result from the modules' C entry points one by one
    h = svdq.svdq_linear_w4a4(x.reshape(192, 256), model.up.layer(), model.up.bias,
                              y_dtype=torch.bfloat16)
    d = svdq.svdq_linear_w4a4_gelu(h, model.down.layer(), model.down.bias,
                                   y_dtype=torch.bfloat16)
    g = svdq.awq_linear_w4a16(x.reshape(192, 256), dict(q=model.gate.q, scales=model.gate.scales,
                                                        zeros=model.gate.zeros, N=256, K=256,
                                                        group=64), model.gate.bias.to(torch.bfloat16))
    assert torch.equal(y.reshape(192, 256), d + g)
    path = str(tmp_path / "mlp.safetensors")
    L.save_quantized(model, path)
    fresh = _mlp(99)
    fresh.act = nn.Identity()
    L.load_quantized(fresh, path, device="cuda")
    with torch.no_grad():
        assert torch.equal(fresh(x), y)


def test_fold_lora_on_module():
    print("SVDQLinear.fold_lora 64x256 -> 128", flush=True)
    lin = _linear(256, 128, 6)
    mod = L.SVDQLinear.from_linear(lin, None, rank=16)
    x = _x(64, 256, 7)
    x = x.float()
    y0 = mod(x)
    a, b = synth.lora_adapter(128, 256, 8, 0)
    at, bt = torch.from_numpy(a).cuda().to(torch.bfloat16), torch.from_numpy(b).cuda().to(torch.bfloat16)
    mod.fold_lora(at, bt, 2.0)
    assert mod.rank == 32
    y1 = mod(x)
    delta = 2.0 * (x.float() @ at.float().T) @ bt.float().T
    assert ((y1 - y0) - delta).norm() / delta.norm() < 0.02
