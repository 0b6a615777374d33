"""Host-side checks of the nn.Linear shim's file format and bookkeeping (no
GPU work): layers built from CPU tensors survive save_quantized /
load_quantized bit for bit, the header is validated, shapes are checked,
and eligibility follows the kernels' shape rules."""

import json

import pytest
import torch
from torch import nn

from w4a4_quantized_diffusion_amd import linear as L
from w4a4_quantized_diffusion_amd import svdq


def _rand(shape, dtype, g):
    if dtype == torch.float32:
        return torch.randn(shape, generator=g)
    if dtype == torch.int16:
        return torch.randint(-32768, 32767, shape, generator=g, dtype=torch.int32).to(torch.int16)
    return torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)


def _svdq_layer(n, k, rank, prec, g):
    lay = {f: _rand(s, dt, g) for f, (s, dt) in L._shapes_svdq(n, k, rank, prec).items()}
    lay.update(rank=rank, prec=prec, N=n, K=k)
    return lay


def _awq_layer(n, k, g):
    lay = {f: _rand(s, dt, g) for f, (s, dt) in L._shapes_awq(n, k, 64).items()}
    lay.update(N=n, K=k, group=64)
    return lay


class Block(nn.Module):
    def __init__(self):
        super().__init__()
        self.attn = nn.ModuleDict({"qkv": nn.Linear(128, 384), "out": nn.Linear(128, 128)})
        self.mlp = nn.Sequential(nn.Linear(128, 512), nn.GELU("tanh"), nn.Linear(512, 128, bias=False))
        self.norm = nn.LayerNorm(128)


def _quantized_block(g):
    b = Block()
    b.attn["qkv"] = L.SVDQLinear(_svdq_layer(384, 128, 32, svdq.INT4, g), torch.randn(384, generator=g))
    b.attn["out"] = L.AWQLinear(_awq_layer(128, 128, g), torch.randn(128, generator=g))
    b.mlp[0] = L.SVDQLinear(_svdq_layer(512, 128, 16, svdq.NVFP4, g), None)
    b.mlp[2] = L.SVDQLinear(_svdq_layer(128, 512, 0, svdq.INT4, g), None, gelu_input=True)
    return b


def test_save_load_roundtrip(tmp_path):
    g = torch.Generator().manual_seed(0)
    q = _quantized_block(g)
    path = str(tmp_path / "block.safetensors")
    names = L.save_quantized(q, path)
    assert sorted(names) == ["attn.out", "attn.qkv", "mlp.0", "mlp.2"]
    fresh = Block()
    assert sorted(L.load_quantized(fresh, path)) == sorted(names)
    for name in names:
        a, b = q.get_submodule(name), fresh.get_submodule(name)
        assert type(a) is type(b)
        assert a.extra_repr() == b.extra_repr()
        for buf_name, buf in a.named_buffers():
            other = getattr(b, buf_name)
            assert buf.dtype == other.dtype and torch.equal(buf, other), (name, buf_name)
    assert isinstance(fresh.norm, nn.LayerNorm) and isinstance(fresh.mlp[1], nn.GELU)
    assert fresh.mlp[2].gelu_input and fresh.mlp[2].rank == 0
    assert fresh.mlp[0].prec == svdq.NVFP4 and fresh.mlp[0].bias is None


def test_header_checked(tmp_path):
    from safetensors.torch import save_file
    g = torch.Generator().manual_seed(1)
    q = _quantized_block(g)
    path = str(tmp_path / "a.safetensors")
    L.save_quantized(q, path)
    from safetensors import safe_open
    with safe_open(path, framework="pt") as f:
        meta = json.loads(f.metadata()["svdq"])
        tensors = {k: f.get_tensor(k) for k in f.keys()}
    assert meta["format"] == L.FORMAT and meta["layers"]["attn.qkv"]["rank"] == 32
    bad = dict(meta, version=L.VERSION + 1)
    save_file(tensors, str(tmp_path / "v.safetensors"), metadata={"svdq": json.dumps(bad)})
    with pytest.raises(ValueError, match="is not"):
        L.load_quantized(Block(), str(tmp_path / "v.safetensors"))
    save_file(tensors, str(tmp_path / "n.safetensors"))
    with pytest.raises(ValueError, match="no svdq header"):
        L.load_quantized(Block(), str(tmp_path / "n.safetensors"))
    # a header whose shapes do not match the stored tensors
    wrong = json.loads(json.dumps(meta))
    wrong["layers"]["attn.qkv"]["N"] = 400
    save_file(tensors, str(tmp_path / "w.safetensors"), metadata={"svdq": json.dumps(wrong)})
    with pytest.raises(ValueError, match="expected"):
        L.load_quantized(Block(), str(tmp_path / "w.safetensors"))
    # a missing tensor
    t2 = {k: v for k, v in tensors.items() if k != "mlp.0.wscales"}
    save_file(t2, str(tmp_path / "m.safetensors"), metadata={"svdq": json.dumps(meta)})
    with pytest.raises(ValueError, match="missing tensor mlp.0.wscales"):
        L.load_quantized(Block(), str(tmp_path / "m.safetensors"))


def test_layer_shapes_validated():
    g = torch.Generator().manual_seed(2)
    lay = _svdq_layer(64, 128, 16, svdq.INT4, g)
    lay["wscales"] = torch.zeros(2, 65)
    with pytest.raises(ValueError, match="wscales"):
        L.SVDQLinear(lay)
    aw = _awq_layer(64, 128, g)
    aw["zeros"] = aw["zeros"].to(torch.float32)
    with pytest.raises(ValueError, match="zeros"):
        L.AWQLinear(aw)


def test_eligibility_and_rank_check():
    assert L.eligible(nn.Linear(3072, 12288), 32)
    assert not L.eligible(nn.Linear(100, 128))          # K not a multiple of 64
    assert not L.eligible(nn.Linear(128, 40))           # N not a multiple of 16
    assert not L.eligible(nn.Linear(64, 16), 32)        # rank above min(N, K)
    with pytest.raises(ValueError, match="rank"):
        L.quantize_linears(Block(), rank=24)
