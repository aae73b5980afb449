"""The autograd wrapper runs the library's backward: its gradients are the
hlq_linear_backward outputs bit for bit (same call on the same ACBP codes),
within the parity bar of the oracle, and what it keeps for the backward is
the INT4 codes of x, not x."""
import numpy as np
import pytest

import oracle as o
from hadamard_rank_linear_amd import workloads as wl
from parity_util import host_f32, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


@pytest.mark.parametrize("name,T", [("tiny", 256), ("vitb_qkv", 1056)])
def test_wrapper_gradients_match_library_and_oracle(name, T):
    import torch
    import hadamard_rank_linear_amd as h
    from hadamard_rank_linear_amd.autograd import hlq_linear
    cfg = wl.BY_NAME[name].with_tokens(T)
    _say(f"autograd {cfg.name} T={T}")
    inp = wl.make_inputs(cfg)
    x = to_device(inp["x"], cfg.dtype).requires_grad_(True)
    w = to_device(inp["w"], cfg.dtype).requires_grad_(True)
    gy = to_device(inp["gy"], cfg.dtype)
    y = hlq_linear(x, w, cfg.block, cfg.rank, cfg.gx_mode, cfg.gw_mode, cfg.reduction)
    assert y.shape == (cfg.T, cfg.O)
    y.backward(gy)
    codes, scales = h.hlq_compress_act(x.detach())
    g_x, g_w = h.hlq_linear_backward(gy, codes, scales, w.detach(), cfg.block, cfg.rank,
                                     cfg.gx_mode, cfg.gw_mode, cfg.reduction)
    torch.cuda.synchronize()
    assert torch.equal(x.grad, g_x.to(x.dtype)) and torch.equal(w.grad, g_w.to(w.dtype))
    oc, os_ = o.acbp_pack(host_f32(inp["x"], cfg.dtype))
    ref = o.linear_backward(host_f32(inp["gy"], cfg.dtype), oc, os_, host_f32(inp["w"], cfg.dtype),
                            cfg.block, cfg.rank, cfg.gx_mode, cfg.gw_mode, cfg.reduction)
    assert o.rel_fro(g_x.cpu().numpy(), ref["g_x"]) <= 1e-5
    assert o.rel_fro(g_w.cpu().numpy(), ref["g_w"]) <= 1e-5


def test_module_keeps_codes_and_flattens_tokens():
    import torch
    from hadamard_rank_linear_amd.autograd import HLQLinear
    _say("autograd module, 3-d input")
    torch.manual_seed(0)
    layer = HLQLinear(64, 48, block=16, rank=4, device="cuda", dtype=torch.float32)
    x = torch.randn(4, 32, 64, device="cuda", requires_grad=True)
    saved = []

    def pack(t):
        saved.append((t.dtype, tuple(t.shape)))
        return t

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        y = layer(x)
    assert y.shape == (4, 32, 48)
    assert (torch.uint8, (128, 32)) in saved            # INT4 codes of x, two per byte
    assert all(s != (torch.float32, (128, 64)) for s in saved)
    y.sum().backward()
    torch.cuda.synchronize()
    assert x.grad.shape == x.shape and layer.weight.grad.shape == (48, 64)
    assert torch.isfinite(x.grad).all() and torch.isfinite(layer.weight.grad).all()
