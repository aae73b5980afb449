"""Synthetic error study of the ablation variants: for every layer config and
every variant of each path (hlq_linear_backward_ablation), the relative
Frobenius error of g_x and g_w against the full-precision products
g_y . w and g_y^T . x (fp64, on the GPU, from the stored inputs before ACBP).

The pages report these ablations as accuracies of ResNet50 trained on
CIFAR100 ("HOT: Hadamard-based Optimized Training", scime.ai summary,
"Measured effects"); with no dataset here the study measures what the
variants do to the gradients of the seeded synthetic layers instead.

    python -m hadamard_rank_linear_amd.ablation_study      (needs the GPU)
"""
from __future__ import annotations

import sys

import numpy as np


def _dev(a, dtype):
    import torch
    if dtype == 1:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _rel_fro(a, b):
    import torch
    d = torch.linalg.norm((a.double() - b).flatten())
    n = torch.linalg.norm(b.flatten())
    return float(d / n) if float(n) > 0 else 0.0


def study(configs=None):
    import torch
    import hadamard_rank_linear_amd as h
    from hadamard_rank_linear_amd import workloads as wl
    rows = []
    for cfg in configs or wl.LAYERS:
        inp = wl.make_inputs(cfg)
        gy, x, w = (_dev(inp[k], cfg.dtype) for k in ("gy", "x", "w"))
        codes, scales = h.hlq_compress_act(x)
        ref_x = gy.double() @ w.double()
        ref_w = gy.double().t() @ x.double()
        if cfg.reduction == wl.MEAN:
            ref_w = ref_w / cfg.T
        for v, name in enumerate(h.VARIANT_NAMES):
            g_x, g_w = h.hlq_linear_backward_ablation(gy, codes, scales, w, cfg.block, cfg.rank,
                                                      v, v, cfg.gx_mode, cfg.gw_mode,
                                                      cfg.reduction)
            rows.append((cfg.name, name, _rel_fro(g_x, ref_x), _rel_fro(g_w, ref_w)))
        del ref_x, ref_w
        torch.cuda.empty_cache()
    return rows


def main():
    rows = study()
    print("| layer | variant | g_x rel. error | g_w rel. error |")
    print("|---|---|---:|---:|")
    for layer, name, ex, ew in rows:
        print(f"| {layer} | {name} | {ex:.4f} | {ew:.4f} |")
    sys.stdout.flush()


if __name__ == "__main__":
    main()
