"""GPU parity of the ablation variants (hlq_linear_backward_ablation) with
the oracle's linear_backward_variant: INT32 sums bit-exact, g_x and g_w within
relative Frobenius error 1e-5 (element-wise 1e-6 where no expansion sums
several products), and the method's own variants equal to the backward."""
import dataclasses

import numpy as np
import pytest

import oracle as o
from hadamard_rank_linear_amd import workloads as wl
from parity_util import ELEM_TOL, FRO_TOL, TINY, host_f32, to_device

pytestmark = pytest.mark.gpu
NAMES = ("hq4", "q4", "hla8_int", "hla8_ext")


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


CASES = [
    # (config, variant index per path, modes)
    (wl.BY_NAME["tiny"], 0, 0, 0, 0), (wl.BY_NAME["tiny"], 1, 1, 1, 1),
    (wl.BY_NAME["tiny"], 2, 2, 0, 1), (wl.BY_NAME["tiny"], 3, 3, 0, 0),
    (wl.BY_NAME["tiny"], 3, 3, 1, 1), (wl.BY_NAME["tiny"], 1, 0, 0, 0),
    (wl.BY_NAME["vitb_qkv"].with_tokens(1040), 3, 1, 0, 0),
    (wl.BY_NAME["vitb_fc2"].with_tokens(1056), 1, 3, 0, 0),
    (wl.BY_NAME["vitb_qkv"].with_tokens(1040), 2, 0, 1, 0),
]


@pytest.mark.parametrize("cfg,vx,vw,gxm,gwm", CASES,
                         ids=[f"{c.name}-{NAMES[a]}-{NAMES[b]}-{m}{n}" for c, a, b, m, n in CASES])
def test_variant_parity(cfg, vx, vw, gxm, gwm):
    import torch
    import hadamard_rank_linear_amd as h
    _say(f"ablation {cfg.name} T={cfg.T} gx={NAMES[vx]} gw={NAMES[vw]} modes=({gxm},{gwm})")
    inp = wl.make_inputs(cfg)
    codes, scales = o.acbp_pack(host_f32(inp["x"], cfg.dtype))
    ref = o.linear_backward_variant(host_f32(inp["gy"], cfg.dtype), codes, scales,
                                    host_f32(inp["w"], cfg.dtype), cfg.block, cfg.rank,
                                    NAMES[vx], NAMES[vw], gxm, gwm, cfg.reduction)
    gy, w = to_device(inp["gy"], cfg.dtype), to_device(inp["w"], cfg.dtype)
    c = torch.from_numpy(codes).cuda()
    s = torch.from_numpy(scales).cuda()
    g_x, g_w, ax, aw = h.hlq_linear_backward_ablation(gy, c, s, w, cfg.block, cfg.rank, vx, vw,
                                                      gxm, gwm, cfg.reduction, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(ax.cpu().numpy().astype(np.int64), ref["acc_x"]), "acc_x differs"
    assert np.array_equal(aw.cpu().numpy().astype(np.int64), ref["acc_w"]), "acc_w differs"
    for name, got, want, expanded in (("g_x", g_x, ref["g_x"], vx == 3),
                                      ("g_w", g_w, ref["g_w"], vw == 3)):
        got = got.cpu().numpy()
        assert np.isfinite(got).all()
        e = o.rel_fro(got, want)
        assert e <= FRO_TOL, f"{name} relative Frobenius error {e:.3e}"
        if not expanded:
            m = o.max_rel_err(got, want, TINY)
            assert m <= ELEM_TOL, f"{name} element-wise relative error {m:.3e}"
    _say("ok")


def test_method_variants_equal_the_backward():
    # hq4 on g_x and internal HLA on g_w through the ablation kernels give the
    # backward's own g_x and g_w bit for bit (same integer sums, same epilogue)
    import torch
    import hadamard_rank_linear_amd as h
    cfg = dataclasses.replace(wl.BY_NAME["vitb_qkv"].with_tokens(528), gw_mode=0)
    _say("ablation hq4 / hla8_int against hlq_linear_backward")
    inp = wl.make_inputs(cfg)
    gy, x, w = (to_device(inp[k], cfg.dtype) for k in ("gy", "x", "w"))
    codes, scales = h.hlq_compress_act(x)
    a_x, a_w = h.hlq_linear_backward_ablation(gy, codes, scales, w, cfg.block, cfg.rank, 0, 2,
                                              cfg.gx_mode, cfg.gw_mode, cfg.reduction)
    b_x, b_w = h.hlq_linear_backward(gy, codes, scales, w, cfg.block, cfg.rank, cfg.gx_mode,
                                     cfg.gw_mode, cfg.reduction)
    torch.cuda.synchronize()
    assert np.array_equal(a_x.cpu().numpy().view(np.uint32), b_x.cpu().numpy().view(np.uint32))
    assert np.array_equal(a_w.cpu().numpy().view(np.uint32), b_w.cpu().numpy().view(np.uint32))
