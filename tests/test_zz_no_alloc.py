"""hlq_linear_backward_noalloc: the backward with the library's static scratch
array instead of a caller workspace, called through the raw C ABI, against
hlq_linear_backward on the same inputs (bit-identical g_x and g_w), on two
calls in a row, the second with a smaller layer.  Plus the host-side refusal
of a shape that does not fit the array."""
import ctypes

import numpy as np
import pytest

from hadamard_rank_linear_amd import workloads as wl
from parity_util import to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def _raw_noalloc(lib, gy, codes, scales, w, cfg, g_x, g_w):
    import torch
    P = ctypes.c_void_p
    return lib.hlq_linear_backward_noalloc(
        P(gy.data_ptr()), 0 if gy.dtype == torch.float32 else 1, P(codes.data_ptr()),
        P(scales.data_ptr()), P(w.data_ptr()), 0 if w.dtype == torch.float32 else 1,
        cfg.T, cfg.I, cfg.O, cfg.block, cfg.rank, cfg.gx_mode, cfg.gw_mode, cfg.reduction,
        P(g_x.data_ptr()), P(g_w.data_ptr()), P(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    import hadamard_rank_linear_amd as h
    lib = h.lib_handle()
    # first a larger layer, then a smaller one: the second call must not see
    # anything of the first in the shared array
    for cfg in (wl.BY_NAME["vitb_qkv"].with_tokens(1040), wl.BY_NAME["tiny"]):
        _say(f"noalloc {cfg.name} T={cfg.T} I={cfg.I} O={cfg.O}")
        inp = wl.make_inputs(cfg)
        gy, x, w = (to_device(inp[k], cfg.dtype) for k in ("gy", "x", "w"))
        codes, scales = h.hlq_compress_act(x)
        ref_x, ref_w = h.hlq_linear_backward(gy, codes, scales, w, cfg.block, cfg.rank,
                                             cfg.gx_mode, cfg.gw_mode, cfg.reduction)
        g_x = torch.full((cfg.T, cfg.I), float("nan"), device="cuda")
        g_w = torch.full((cfg.O, cfg.I), float("nan"), device="cuda")
        assert _raw_noalloc(lib, gy, codes, scales, w, cfg, g_x, g_w) == 0
        torch.cuda.synchronize()
        assert np.array_equal(g_x.cpu().numpy().view(np.uint32), ref_x.cpu().numpy().view(np.uint32))
        assert np.array_equal(g_w.cpu().numpy().view(np.uint32), ref_w.cpu().numpy().view(np.uint32))


def test_noalloc_refuses_shapes_beyond_the_array():
    import torch
    import hadamard_rank_linear_amd as h
    lib = h.lib_handle()
    # a layer whose intermediates exceed the array: refused on the host, no launch
    cfg = wl.BY_NAME["llama3_8b_down"].with_tokens(16384)
    assert h.hlq_linear_backward_workspace_size(cfg.T, cfg.I, cfg.O, cfg.block, cfg.rank) > \
        h.HLQ_NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    P = ctypes.c_void_p(buf.data_ptr())
    got = lib.hlq_linear_backward_noalloc(P, 1, P, P, P, 1, cfg.T, cfg.I, cfg.O, cfg.block,
                                          cfg.rank, 0, 0, 0, P, P, None)
    assert got == 9
    torch.cuda.synchronize()
    assert (buf == 0).all()
