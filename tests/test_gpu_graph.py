"""The backward enqueues only kernels (no allocation, no memset, no host
synchronisation), so it can be captured in a HIP graph.  The captured graph is
replayed several times with the program's own eager work and synchronisations
between the replays; every replay must reproduce the eager result bit for bit."""
import numpy as np
import pytest

from hadamard_rank_linear_amd import workloads as wl
from parity_util import to_device

pytestmark = pytest.mark.gpu


def test_backward_graph_replays_match_eager():
    import torch
    import hadamard_rank_linear_amd as h
    cfg = wl.BY_NAME["vitb_qkv"].with_tokens(1056)
    print(f"\n[gpu-case] graph capture {cfg.name} T={cfg.T}", flush=True)
    inp = wl.make_inputs(cfg)
    gy, x, w = (to_device(inp[k], cfg.dtype) for k in ("gy", "x", "w"))
    codes, scales = h.hlq_compress_act(x)
    ws = torch.zeros((h.hlq_linear_backward_workspace_size(cfg.T, cfg.I, cfg.O, cfg.block,
                                                           cfg.rank),),
                     dtype=torch.uint8, device="cuda")
    g_x = torch.empty((cfg.T, cfg.I), dtype=torch.float32, device="cuda")
    g_w = torch.empty((cfg.O, cfg.I), dtype=torch.float32, device="cuda")

    def run():
        h.hlq_linear_backward(gy, codes, scales, w, cfg.block, cfg.rank, cfg.gx_mode,
                              cfg.gw_mode, cfg.reduction, g_x=g_x, g_w=g_w, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref_x, ref_w = g_x.clone(), g_w.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        g_x.fill_(float("nan"))
        g_w.fill_(float("nan"))
        ws.fill_(0xA5)                    # stale intermediates must not matter
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert np.array_equal(g_x.cpu().numpy().view(np.uint32), ref_x.cpu().numpy().view(np.uint32)), rep
        assert np.array_equal(g_w.cpu().numpy().view(np.uint32), ref_w.cpu().numpy().view(np.uint32)), rep
