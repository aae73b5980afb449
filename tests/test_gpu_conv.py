"""GPU parity of the convolution backward (implicit GEMMs: im2col gathered
by the g_w path's x loader, col2im as the input-gradient GEMM's sum over the
taps) against the oracle's convolution form, on the same seeded inputs.

Bar as for the linear layer: ACBP bytes and scales, every operand's codes and
scales, both GEMMs' INT32 accumulators bit-exact; g_x and g_w within relative
Frobenius error 1e-5 and element-wise relative error 1e-6."""
import dataclasses

import numpy as np
import pytest

import oracle as o
from hadamard_rank_linear_amd import workloads as wl
from parity_util import GpuRun, compare, host_f32, to_device, unplane

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def _run(cfg, seed=0):
    import torch
    import hadamard_rank_linear_amd as h
    _say(f"conv {cfg.name} N={cfg.N} H={cfg.H} W={cfg.W} C={cfg.C} O={cfg.O} R={cfg.R} "
         f"S={cfg.S} stride={cfg.stride} pad={cfg.pad} n={cfg.block} r={cfg.rank} "
         f"modes=({cfg.gx_mode},{cfg.gw_mode}) red={cfg.reduction} dtype={cfg.dtype}")
    inp = wl.make_conv_inputs(cfg, seed=seed)
    x32 = host_f32(inp["x"], cfg.dtype)
    ocodes, oscales = o.acbp_pack(x32)
    ref = o.conv_backward(host_f32(inp["gy"], cfg.dtype), ocodes, oscales,
                          host_f32(inp["w"], cfg.dtype), cfg.N, cfg.H, cfg.W, cfg.C, cfg.R,
                          cfg.S, cfg.stride, cfg.pad, cfg.block, cfg.rank, cfg.gx_mode,
                          cfg.gw_mode, cfg.reduction)
    gy = to_device(inp["gy"], cfg.dtype)
    x = to_device(inp["x"], cfg.dtype)
    w = to_device(inp["w"], cfg.dtype)
    codes, scales = h.hlq_compress_act(x)
    geo = (cfg.N, cfg.H, cfg.W, cfg.C, cfg.O, cfg.R, cfg.S, cfg.stride, cfg.pad, cfg.block,
           cfg.rank)
    ws = torch.zeros((h.hlq_conv_backward_workspace_size(*geo),), dtype=torch.uint8,
                     device="cuda")
    g_x, g_w = h.hlq_conv_backward(gy, codes, scales, w, cfg.N, cfg.H, cfg.W, cfg.C, cfg.R,
                                   cfg.S, cfg.stride, cfg.pad, cfg.block, cfg.rank, cfg.gx_mode,
                                   cfg.gw_mode, cfg.reduction, workspace=ws)
    acc_x, acc_w = h.hlq_conv_gemm_acc(ws, *geo)
    torch.cuda.synchronize()
    lay = h.hlq_workspace_layout_query(cfg.T, cfg.I, cfg.O, cfg.block, cfg.rank)
    wsh = ws.cpu().numpy()

    def region(off, count, dt):
        return wsh[off: off + count * np.dtype(dt).itemsize].view(dt)

    T, I, O = cfg.T, cfg.I, cfg.O
    kxb, kwb = lay["kx_pitch"], lay["kw_pitch"]
    n_gw = O if cfg.gw_mode == wl.PER_TOKEN else 1
    n_xw = I if cfg.gw_mode == wl.PER_TOKEN else 1
    inter = dict(
        q_gy_packed=unplane(region(lay["q_gy"], T * kxb, np.uint8), T, kxb, 96),
        s_gy=region(lay["s_gy"], 1, np.float32).copy(),
        q_w_packed=unplane(region(lay["q_w"], I * kxb, np.uint8), I, kxb, 96),
        s_w=region(lay["s_w"], 1, np.float32).copy(),
        q_gyl_stored=unplane(region(lay["q_gyl"], O * kwb, np.int8), O, kwb, 64),
        s_gyl=region(lay["s_gyl"], n_gw, np.float32).copy(),
        q_xl_stored=unplane(region(lay["q_xl"], I * kwb, np.int8), I, kwb, 64),
        s_xl=region(lay["s_xl"], n_xw, np.float32).copy(),
        kxb=kxb, kwb=kwb, t_low=lay["t_low"])
    # the input-gradient GEMM and the g_w GEMM are the only GEMM launches here
    ax, aw = acc_x.cpu().numpy(), acc_w.cpu().numpy()
    inter.update(acc_x=ax, acc_w=aw, acc_x1=ax, acc_w1=aw)
    gpu = GpuRun(codes.cpu().numpy(), scales.cpu().numpy(), g_x.cpu().numpy(),
                 g_w.cpu().numpy(), inter)
    ex, ew = compare(cfg, gpu, ocodes, oscales, ref)
    _say(f"ok rel_fro g_x={ex:.2e} g_w={ew:.2e}")


SMALL = [
    wl.CONV_BY_NAME["small_stride2_pad1"],
    # stride 1, pad 1, 24 channels: 128-column tiles straddle the taps
    dataclasses.replace(wl.CONV_BY_NAME["small_stride2_pad1"], name="s1_pad1_c24", N=4, H=10,
                        W=10, C=24, O=48, stride=1, pad=1, dtype=wl.BF16, gw_mode=wl.PER_TENSOR,
                        index=22),
    # 1x1, stride 2, no padding
    dataclasses.replace(wl.CONV_BY_NAME["small_stride2_pad1"], name="k1_s2", N=2, H=16, W=16,
                        C=64, O=64, R=1, S=1, stride=2, pad=0, index=23),
    # 5x3 taps, pad 2, mean reduction, block 32
    dataclasses.replace(wl.CONV_BY_NAME["small_stride2_pad1"], name="k5x3_pad2_mean", N=2, H=8,
                        W=16, C=32, O=64, R=5, S=3, stride=1, pad=2, block=32, rank=4,
                        reduction=wl.MEAN, index=24),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_conv_small(cfg):
    _run(cfg)


def test_conv_resnet50_stage3_full_size():
    _run(wl.CONV_BY_NAME["resnet50_s3_conv3x3"])
