#!/usr/bin/env python3
"""Per-layer HLQ/HOT backward latency on one MI355X.

One step = one full backward of the layer (hlq_linear_backward: every launch
of the hot path) on inputs already resident in HBM.  The ACBP compression of x
happens at forward time; it is timed separately (as one more launch of the
instrumented pass below) and reported as acbp_us.

Timing: W untimed warm-up steps, then K steps bracketed by
torch.cuda.synchronize(); the steps rotate over several copies of the
inputs/outputs/workspace whose total exceeds the 256 MB last-level cache, so
every step reads its operands from HBM.  A second, instrumented pass records
HIP events around each launch step (same stream, same rotation) to get
per-kernel durations (less the interval of an empty step, the cost of the
event itself); the longest one is reported against its roofline.

The CPU baseline is the oracle (numpy) running the same layer once on one host
thread.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA
FP6_PEAK_TOPS = 10100.0        # MI355X dense FP6 / FP4 MFMA (the g_x product's unit)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
LLC_BYTES = 256 << 20
METRIC = "per-layer BP latency (us) + effective TOPS & % roofline, ViT-B qkv/fc2 shape"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_costs(cfg, dt_bytes):
    """Algorithmic (ops, bytes) per launch step: each input read once, each
    output written once (partial maxima and scale vectors included)."""
    T, I, O, Tl = cfg.T, cfg.I, cfg.O, cfg.Tl
    gy = T * O * dt_bytes
    w = O * I * dt_bytes
    xc = T * I // 2 + 4 * T
    # partial maxima: H.g_y rows per 128-channel chunk, low-rank g_y columns per
    # token span (256 tokens on the register path: bf16 g_y with n <= 64, else
    # 128), low-rank x columns per 128 tokens, H.w columns per 128 channels
    gy_rows = 256 if (dt_bytes == 2 and cfg.block <= 64) else 128
    parts = 4 * (T * -(-O // 128) + O * -(-T // gy_rows) + I * -(-T // 128) + I * -(-O // 128))
    return {
        "tr_max": (0, gy + xc + w + parts),
        "tr_reduce": (0, parts + 4 * (T + O + 2 * I)),
        "tr_quant": (0, gy + xc + w + T * O // 2 + I * O // 2 + O * Tl + I * Tl
                     + 4 * (T + O + 2 * I)),
        # both GEMMs run as one launch (k_gemm_pair) when a step holds both
        "gemm": (2 * T * I * O + 2 * O * I * Tl,
                 T * O // 2 + I * O // 2 + 4 * T + 4 * I + 4 * T * I
                 + O * Tl + I * Tl + 4 * O + 4 * I + 4 * O * I),
    }


KERNEL_SOURCES = ("hlq_device.h", "hlq_internal.h", "hlq_tr.hip", "hlq_gemm.hip", "hlq_acbp.hip")


def kernel_source_sha():
    """SHA-256 over the kernel sources (in a fixed order): a counter record
    taken for other sources is not reported."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "hadamard_rank_linear_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-kernel calibrated), or None when
    there is none or the kernel source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernels_source_sha256") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(nbytes=256 << 20, reps=5):
    """Plain device-to-device copies of known size: their FETCH_SIZE and
    WRITE_SIZE in a counter run give the scale of those counters."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


def mfma_peak_tops(cfg, kname):
    """Matrix-core peak of a launch step: the g_x product runs on the FP6
    matrix cores (its INT4 codes stored as FP6, 10.1 POP/s), the g_w product
    on the INT8 ones (5.0 POP/s); the pair's peak is their time-weighted mean
    (total ops over the sum of each product's ideal time)."""
    if kname != "gemm":
        return INT8_PEAK_TOPS
    ox, ow = 2 * cfg.T * cfg.I * cfg.O, 2 * cfg.O * cfg.I * cfg.Tl
    return (ox + ow) / (ox / FP6_PEAK_TOPS + ow / INT8_PEAK_TOPS)


def ideal_us(ops, nbytes, peak_tops=INT8_PEAK_TOPS):
    t_mfma = ops / (peak_tops * 1e12) * 1e6
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
    return max(t_mfma, t_hbm), ("mfma" if t_mfma > t_hbm else "hbm")


class LayerSets:
    """Rotating device copies of one layer's inputs, outputs and workspace."""

    def __init__(self, cfg, inp, nsets):
        import torch
        import hadamard_rank_linear_amd as h
        self.cfg = cfg
        dev = torch.device("cuda:0")
        bf = cfg.dtype == 1
        import numpy as np

        def dev_t(a):
            if bf:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        gy0, x0, w0 = dev_t(inp["gy"]), dev_t(inp["x"]), dev_t(inp["w"])
        codes0, scales0 = h.hlq_compress_act(x0)
        self.x0 = x0
        ws_bytes = h.hlq_linear_backward_workspace_size(cfg.T, cfg.I, cfg.O, cfg.block, cfg.rank)
        self.sets = []
        for _ in range(nsets):
            self.sets.append(dict(
                gy=gy0.clone(), x=x0.clone(), codes=codes0.clone(), scales=scales0.clone(),
                w=w0.clone(),
                g_x=torch.empty((cfg.T, cfg.I), dtype=torch.float32, device=dev),
                g_w=torch.empty((cfg.O, cfg.I), dtype=torch.float32, device=dev),
                ws=torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)))
        self.bytes_per_set = sum(t.numel() * t.element_size() for t in self.sets[0].values())
        del gy0, w0
        torch.cuda.synchronize()

    def acbp(self, i):
        import hadamard_rank_linear_amd as h
        s = self.sets[i % len(self.sets)]
        h.hlq_compress_act(s["x"], s["codes"], s["scales"])

    def run(self, i, steps=None):
        import hadamard_rank_linear_amd as h
        s = self.sets[i % len(self.sets)]
        c = self.cfg
        if steps == "acbp":
            self.acbp(i)
            return
        h.hlq_linear_backward(s["gy"], s["codes"], s["scales"], s["w"], c.block, c.rank,
                              c.gx_mode, c.gw_mode, c.reduction, g_x=s["g_x"], g_w=s["g_w"],
                              workspace=s["ws"], steps=steps)


def time_layer(cfg, inp, steps, warmup, per_kernel=True):
    import torch
    import hadamard_rank_linear_amd as h
    probe = LayerSets(cfg, inp, 1)
    nsets = max(2, -(-2 * LLC_BYTES // probe.bytes_per_set))
    del probe
    torch.cuda.empty_cache()
    sets = LayerSets(cfg, inp, nsets)
    log(f"{cfg.name}: {nsets} rotating sets of {sets.bytes_per_set / 1e6:.1f} MB")
    for i in range(warmup):
        sets.run(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        sets.run(i)
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    gpu_ms = ev0.elapsed_time(ev1)
    res = dict(wall_ms_per_step=wall_ms / steps, gpu_ms_per_step=gpu_ms / steps, nsets=nsets)

    if per_kernel:
        # Distribution of single-step latencies: an event before every step of
        # a run queued behind a spin kernel (no host gap inside an interval);
        # the empty-interval cost measured below is subtracted.
        n_dist = min(max(steps, 20), 100)
        cal0 = torch.cuda.Event(enable_timing=True)
        cal1 = torch.cuda.Event(enable_timing=True)
        cal0.record()
        torch.cuda._sleep(1 << 20)
        cal1.record()
        torch.cuda.synchronize()
        cyc_per_us = (1 << 20) / max(cal0.elapsed_time(cal1) * 1e3, 1e-3)
        torch.cuda._sleep(int((2000 + n_dist * 150) * cyc_per_us))
        evs = []
        for i in range(n_dist):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            evs.append(e)
            sets.run(i)
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        evs.append(e)
        torch.cuda.synchronize()
        res["step_event_us"] = [a.elapsed_time(b) * 1e3 for a, b in zip(evs, evs[1:])]

        # In-pipeline per-kernel durations: an event before every launch step
        # of every step, enqueued while a spin kernel holds the GPU so that the
        # queue is full and no launch gap lands inside a measured interval.
        # launch units as the full backward runs them: the two GEMM steps
        # together are one launch
        # The "empty" unit launches nothing: its interval is the cost of one
        # event record in the queue, subtracted from the others.
        # ACBP (forward time, hlq_compress_act) is timed the same way
        units = [("tr_max", 1 << 0), ("tr_reduce", 1 << 1), ("tr_quant", 1 << 2),
                 ("gemm", (1 << 3) | (1 << 4)), ("acbp", "acbp"), ("empty", 0)]
        active = list(range(len(units)))
        n_inst = min(steps, 20)
        cal0 = torch.cuda.Event(enable_timing=True)
        cal1 = torch.cuda.Event(enable_timing=True)
        cal0.record()
        torch.cuda._sleep(1 << 20)
        cal1.record()
        torch.cuda.synchronize()
        cycles_per_us = (1 << 20) / max(cal0.elapsed_time(cal1) * 1e3, 1e-3)
        hold_us = 2000 + n_inst * len(active) * 60
        torch.cuda._sleep(int(hold_us * cycles_per_us))
        marks = []
        for i in range(n_inst):
            for k in active:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                marks.append((k, e))
                sets.run(i, steps=units[k][1])
        end = torch.cuda.Event(enable_timing=True)
        end.record()
        torch.cuda.synchronize()
        marks.append((None, end))
        acc = {k: 0.0 for k in active}
        for (k, a), (_, b) in zip(marks, marks[1:]):
            acc[k] += a.elapsed_time(b)
        raw = {units[k][0]: acc[k] / n_inst * 1e3 for k in active}
        empty = raw.pop("empty")
        res["acbp_us"] = max(raw.pop("acbp") - empty, 0.0)
        res["kernels_event_us"] = raw
        res["event_overhead_us"] = empty
        res["kernels_us"] = {k: max(v - empty, 0.0) for k, v in raw.items()}
        import numpy as np
        lat = np.array(res.pop("step_event_us")) - empty
        res["latency_us"] = {"p10": round(float(np.percentile(lat, 10)), 2),
                             "p50": round(float(np.percentile(lat, 50)), 2),
                             "p90": round(float(np.percentile(lat, 90)), 2), "steps": int(lat.size)}
        res["instrumented_steps"] = n_inst
    del sets
    torch.cuda.empty_cache()
    return res


def roofline_of(cfg, kernels_us):
    """Roofline object of the dominant (longest) launch of one backward: its
    algorithmic work per launch over its measured duration, against the bound
    its arithmetic intensity gives (INT8 MFMA or HBM)."""
    dt_bytes = 4 if cfg.dtype == 0 else 2
    costs = step_costs(cfg, dt_bytes)
    kname = max((k for k in kernels_us if k in costs), key=lambda k: kernels_us[k])
    kus = kernels_us[kname]
    ops, nbytes = costs[kname]
    peak = mfma_peak_tops(cfg, kname)
    _, bound = ideal_us(ops, nbytes, peak)
    if bound == "mfma":
        achieved = ops / (kus * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": round(peak, 1),
                "unit": "TOP/s", "frac": round(achieved / peak, 4),
                "peak_parts": {"g_x FP6 (INT4 codes)": FP6_PEAK_TOPS, "g_w INT8": INT8_PEAK_TOPS},
                "frac_of_int8_peak": round(achieved / INT8_PEAK_TOPS, 4)}
    else:
        achieved = nbytes / (kus * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        if ops:  # a product whose ideal HBM time exceeds its ideal matrix-core time
            roof.update(achieved_tops=round(ops / (kus * 1e-6) / 1e12, 1),
                        mfma_peak_tops=round(peak, 1),
                        mfma_frac=round(ops / (kus * 1e-6) / 1e12 / peak, 4))
    roof.update(kernel=kname, kernel_us=round(kus, 2), algorithmic_bytes=nbytes,
                algorithmic_ops=ops, traffic=measured_traffic(cfg.name, kname))
    return roof


def layer_summary(cfg, r):
    """µs per backward, effective TOPS, per-launch times, latency
    percentiles and the dominant launch's roofline of one timed layer."""
    us = r["wall_ms_per_step"] * 1e3
    ops = 2 * cfg.T * cfg.I * cfg.O + 2 * cfg.Tl * cfg.O * cfg.I
    out = {"us": round(us, 2), "effective_tops": round(ops / (us * 1e-6) / 1e12, 1)}
    if "kernels_us" in r:
        out["kernels_us"] = {k: round(v, 2) for k, v in r["kernels_us"].items()}
        out["acbp_us"] = round(r["acbp_us"], 2)
        out["latency_us"] = r["latency_us"]
        out["roofline"] = roofline_of(cfg, r["kernels_us"])
    return out


def time_int8_library_gemm(M, N, K, reps=20):
    """Context, not this library: torch._int_mm (hipBLASLt) INT8 x INT8 ->
    INT32 of an M x K by K x N product, µs per call on resident operands, and
    its fraction of the INT8 peak.  None when the build has no INT8 GEMM."""
    import torch
    try:
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
        b = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda").t()
        for _ in range(3):
            torch._int_mm(a, b)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch._int_mm(a, b)
        e1.record()
        torch.cuda.synchronize()
    except Exception as ex:  # pragma: no cover - depends on the torch build
        return {"error": str(ex)[:120]}
    us = e0.elapsed_time(e1) / reps * 1e3
    tops = 2 * M * N * K / (us * 1e-6) / 1e12
    return {"M": M, "N": N, "K": K, "us": round(us, 2), "tops": round(tops, 1),
            "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}


def time_conv(cfg, steps, warmup):
    """The convolution backward (hlq_conv_backward: implicit GEMMs, no
    im2col / col2im buffer) on rotating device copies: µs per backward and
    effective TOPS (the same integer work as its im2col linear form)."""
    import numpy as np
    import torch
    import hadamard_rank_linear_amd as h
    from hadamard_rank_linear_amd import workloads as wl
    inp = wl.make_conv_inputs(cfg)
    dev = torch.device("cuda:0")

    def dev_t(a):
        if cfg.dtype == wl.BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    geo = (cfg.N, cfg.H, cfg.W, cfg.C, cfg.O, cfg.R, cfg.S, cfg.stride, cfg.pad, cfg.block,
           cfg.rank)
    ws_bytes = h.hlq_conv_backward_workspace_size(*geo)
    gy0, x0, w0 = dev_t(inp["gy"]), dev_t(inp["x"]), dev_t(inp["w"])
    codes0, scales0 = h.hlq_compress_act(x0)
    per_set = (gy0.numel() * gy0.element_size() + codes0.numel() + 4 * scales0.numel()
               + w0.numel() * w0.element_size() + 4 * (x0.numel() + w0.numel()) + ws_bytes)
    n = max(2, -(-2 * LLC_BYTES // per_set))
    sets = [dict(gy=gy0.clone(), codes=codes0.clone(), scales=scales0.clone(), w=w0.clone(),
                 g_x=torch.empty((cfg.N * cfg.H * cfg.W, cfg.C), dtype=torch.float32, device=dev),
                 g_w=torch.empty((cfg.O, cfg.I), dtype=torch.float32, device=dev),
                 ws=torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)) for _ in range(n)]
    del x0

    def run(i):
        st = sets[i % n]
        h.hlq_conv_backward(st["gy"], st["codes"], st["scales"], st["w"], cfg.N, cfg.H, cfg.W,
                            cfg.C, cfg.R, cfg.S, cfg.stride, cfg.pad, cfg.block, cfg.rank,
                            cfg.gx_mode, cfg.gw_mode, cfg.reduction, g_x=st["g_x"],
                            g_w=st["g_w"], workspace=st["ws"])

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    ops = 2 * cfg.T * cfg.I * cfg.O + 2 * cfg.Tl * cfg.O * cfg.I
    del sets
    torch.cuda.empty_cache()
    return {"us": round(us, 2), "effective_tops": round(ops / (us * 1e-6) / 1e12, 1),
            "shape": f"N={cfg.N} H={cfg.H} W={cfg.W} C={cfg.C} O={cfg.O} R={cfg.R} S={cfg.S} "
                     f"stride={cfg.stride} pad={cfg.pad}", "rotating_sets": n}


def time_forward(cfg, inp, steps=20, warmup=5):
    """Forward of the layer (bf16): hlq_linear_forward (the bf16 MFMA product
    with the ACBP codes of x from the same launch) against torch's matmul
    followed by hlq_compress_act, on rotating operand copies.  µs per forward,
    TFLOP/s of the product against the bf16 dense peak."""
    import numpy as np
    import torch
    import hadamard_rank_linear_amd as h
    if cfg.dtype != 1 or cfg.I % 32:
        return None
    dev = torch.device("cuda:0")

    def dev_t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x0, w0 = dev_t(inp["x"]), dev_t(inp["w"])
    per_set = 2 * (x0.numel() + w0.numel() + cfg.T * cfg.O) + cfg.T * cfg.I // 2 + 4 * cfg.T
    n = max(2, -(-2 * LLC_BYTES // per_set))
    sets = [(x0.clone(), w0.clone(), torch.empty((cfg.T, cfg.O), dtype=torch.bfloat16, device=dev),
             torch.empty((cfg.T, cfg.I // 2), dtype=torch.uint8, device=dev),
             torch.empty((cfg.T,), dtype=torch.float32, device=dev)) for _ in range(n)]

    def fused(i):
        x, w, y, c, sc = sets[i % n]
        h.hlq_linear_forward(x, w, y=y, x_codes=c, x_scales=sc)

    def product(i):
        x, w, y, c, sc = sets[i % n]
        h.hlq_linear_forward(x, w, y=y, compress=False)

    def unfused(i):
        x, w, y, c, sc = sets[i % n]
        torch.mm(x, w.t(), out=y)
        h.hlq_compress_act(x, c, sc)

    out = {}
    for name, fn in (("fused_us", fused), ("product_only_us", product),
                     ("torch_matmul_plus_acbp_us", unfused)):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / steps * 1e3, 2)
    flops = 2 * cfg.T * cfg.I * cfg.O
    out["fused_tflops"] = round(flops / (out["fused_us"] * 1e-6) / 1e12, 1)
    out["fused_frac_of_bf16_peak"] = round(out["fused_tflops"] / BF16_PEAK_TFLOPS, 4)
    del sets
    torch.cuda.empty_cache()
    return out


def time_lqs(cfg, inp, reps=10):
    """Layer-wise quantizer selection statistics of one calibration batch
    (hlq_lqs_accumulate: the backward's MAX and reduce launches, an error
    pass, a fold) on the layer's inputs, and the modes the 50% rule picks from
    them.  Algorithmic bytes: the MAX launch reads g_y, w and the ACBP codes
    once; the error pass reads g_y twice (rows along O, columns along T), w
    and the codes once."""
    import numpy as np
    import torch
    import hadamard_rank_linear_amd as h
    dev = torch.device("cuda:0")
    bf = cfg.dtype == 1

    def dev_t(a):
        if bf:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    gy, x, w = dev_t(inp["gy"]), dev_t(inp["x"]), dev_t(inp["w"])
    codes, scales = h.hlq_compress_act(x)
    ws = torch.empty((h.hlq_lqs_workspace_size(cfg.T, cfg.I, cfg.O, cfg.block, cfg.rank),),
                     dtype=torch.uint8, device=dev)
    stats = torch.zeros((16,), dtype=torch.float64, device=dev)
    h.hlq_lqs_accumulate(gy, codes, scales, w, cfg.block, cfg.rank, stats=stats, workspace=ws)
    torch.cuda.synchronize()
    modes = h.hlq_lqs_select(stats)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        h.hlq_lqs_accumulate(gy, codes, scales, w, cfg.block, cfg.rank, stats=stats, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    e = 2 if bf else 4
    once = cfg.O * cfg.I * e + cfg.T * cfg.I // 2 + 4 * cfg.T
    nbytes = (cfg.T * cfg.O * e + once) + (2 * cfg.T * cfg.O * e + once)
    return {"us": round(us, 2), "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "selected_modes": {"gx": "per_token" if modes[0] == 0 else "per_tensor",
                               "gw": "per_token" if modes[1] == 0 else "per_tensor"}}


def time_torch_backward(cfg, inp, dtype_name="bf16", steps=20, warmup=5):
    """Context, not this library: the plain backward of the same layer in
    torch at bf16 or fp32 (g_x = g_y . w and g_w = g_y^T . x, two 2-D matmuls
    on hipBLASLt), µs per layer on rotating operand copies.  The transposed
    operand is the left one of a 2-D product."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype_name == "bf16" else torch.float32

    def dev_t(a):
        if cfg.dtype == 1:
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        return t.to(dev).to(tdt)

    gy0, x0, w0 = dev_t(inp["gy"]), dev_t(inp["x"]), dev_t(inp["w"])
    esz = 2 if tdt == torch.bfloat16 else 4
    per_set = (gy0.numel() + x0.numel() + w0.numel() + cfg.T * cfg.I + cfg.O * cfg.I) * esz
    n = max(2, -(-2 * LLC_BYTES // per_set))
    sets = [(gy0.clone(), x0.clone(), w0.clone(),
             torch.empty((cfg.T, cfg.I), dtype=tdt, device=dev),
             torch.empty((cfg.O, cfg.I), dtype=tdt, device=dev)) for _ in range(n)]

    def step(i):
        gy, x, w, gx, gw = sets[i % n]
        torch.mm(gy, w, out=gx)
        torch.mm(gy.t(), x, out=gw)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    return round((time.perf_counter() - t0) / steps * 1e6, 2)


def per_config_side(steps, warmup):
    """Every other layer config at full size: µs per backward, effective TOPS,
    per-launch event times and the dominant launch's roofline."""
    from hadamard_rank_linear_amd import workloads as wl
    out = {}
    for cfg in wl.LAYERS:
        if cfg.name in ("vitb_qkv", "vitb_fc2"):
            continue
        log(f"side measurement: {cfg.name}")
        out[cfg.name] = layer_summary(cfg, time_layer(cfg, wl.make_inputs(cfg), steps, warmup))
    return out


def cpu_baseline(cfg, inp):
    """The oracle (numpy, as it stands) on the same full layer, once, on one
    host thread: BLAS is held to one thread for the integer GEMMs (fp64
    products), and the transforms and quantizers are single-threaded numpy."""
    import oracle as o
    from threadpoolctl import threadpool_limits
    f = (lambda a: a) if cfg.dtype == 0 else o.bf16_bits_to_f32
    gy, x, w = f(inp["gy"]), f(inp["x"]), f(inp["w"])
    codes, scales = o.acbp_pack(x)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        o.linear_backward(gy, codes, scales, w, cfg.block, cfg.rank, cfg.gx_mode, cfg.gw_mode,
                          cfg.reduction)
        sec = time.perf_counter() - t0
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                       cpu)
    except OSError:
        pass
    return {"value": round(sec * 1e6, 1), "unit": "us", "cores": 1, "kind": "oracle",
            "cpu": cpu, "host_cpus": os.cpu_count(),
            "sample": (f"one full {cfg.name} layer backward (T={cfg.T}, I={cfg.I}, O={cfg.O}) by "
                       f"the numpy oracle on one host thread (BLAS limited to 1 thread for the "
                       f"exact fp64 integer GEMMs); ACBP excluded"),
            "seconds": round(sec, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 300 untimed steps (about 30 ms of ViT-B qkv work): the GPU's clocks
    # settle under load only after some tens of milliseconds; ten warmup
    # steps timed the same 50 steps 10 % slower
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="vitb_qkv")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the side measurements (fc2 layer, LQS statistics)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run 256 MiB device copies (scale of the HBM byte counters)")
    ap.add_argument("--side", choices=("conv", "forward"),
                    help="run only this side measurement (the ResNet-50 stage-3 convolution "
                         "backward, or the forward with fused ACBP on --workload) and print "
                         "its JSON; for profiling")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the HLQ/HOT layer backward here runs on a "
              "single MI355X (no sharding, no collectives); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from hadamard_rank_linear_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.side == "conv":
        c = wl.CONV_BY_NAME["resnet50_s3_conv3x3"]
        print(json.dumps({"side": "conv", "workload": c.name,
                          "result": time_conv(c, args.steps, args.warmup)}), flush=True)
        return
    if args.side == "forward":
        c = wl.BY_NAME[args.workload]
        print(json.dumps({"side": "forward", "workload": c.name,
                          "result": time_forward(c, wl.make_inputs(c), args.steps, args.warmup)}),
              flush=True)
        return

    cfg = wl.BY_NAME[args.workload]
    log(f"generating {cfg.name} inputs")
    inp = wl.make_inputs(cfg)
    res = time_layer(cfg, inp, args.steps, args.warmup)
    lat_us = res["wall_ms_per_step"] * 1e3
    costs = step_costs(cfg, 4 if cfg.dtype == 0 else 2)
    ops_total = 2 * cfg.T * cfg.I * cfg.O + 2 * cfg.Tl * cfg.O * cfg.I
    ideal_total = sum(ideal_us(*costs[k], mfma_peak_tops(cfg, k))[0]
                      for k in res["kernels_us"] if k in costs)

    # dominant kernel against its roofline
    roof = roofline_of(cfg, res["kernels_us"])

    extra = {}
    if not args.no_extra:
        log("layer-wise quantizer selection statistics")
        extra["lqs"] = time_lqs(cfg, inp)
    if not args.no_extra and cfg.name != "vitb_fc2":
        # the other half of the metric's "qkv/fc2 shape": same measurement
        c2 = wl.BY_NAME["vitb_fc2"]
        log("side measurement: vitb_fc2")
        extra["vitb_fc2"] = layer_summary(c2, time_layer(c2, wl.make_inputs(c2),
                                                         max(10, args.steps // 2), args.warmup))
        extra["vitb_fc2_us"] = extra["vitb_fc2"]["us"]
    if not args.no_extra:
        extra["per_config"] = per_config_side(max(10, args.steps // 2), args.warmup)
        log("side measurement: forward with fused ACBP")
        extra["forward"] = time_forward(cfg, inp, warmup=args.warmup)
        log("side measurement: ResNet-50 stage-3 convolution (implicit GEMM)")
        extra["conv"] = {"resnet50_s3_conv3x3": time_conv(
            wl.CONV_BY_NAME["resnet50_s3_conv3x3"], max(10, args.steps // 2), args.warmup)}
        log("context: torch bf16 and fp32 backward of the same layer")
        extra["context_torch_bf16_backward_us"] = time_torch_backward(cfg, inp, "bf16",
                                                                      warmup=args.warmup)
        extra["context_torch_fp32_backward_us"] = time_torch_backward(cfg, inp, "fp32", steps=10,
                                                                      warmup=args.warmup // 4)
        # the library INT8 GEMM on the same two products (g_w: INT8 codes,
        # K = T'; g_x: its INT4 codes as INT8, K = O), for context
        log("context: hipBLASLt INT8 GEMMs of the layer's shapes")
        extra["context_hipblaslt_int8"] = {
            "gemm_gw": time_int8_library_gemm(cfg.O, cfg.I, -(-cfg.Tl // 8) * 8),
            "gemm_gx": time_int8_library_gemm(cfg.T, cfg.I, cfg.O)}

    if args.copy_calib:
        copy_calibration()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(cfg, inp)

    line = {
        "metric": METRIC,
        "value": round(lat_us, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall_ms_per_step"], 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "I": cfg.I, "O": cfg.O,
                   "block": cfg.block, "rank": cfg.rank, "gx_mode": cfg.gx_mode,
                   "gw_mode": cfg.gw_mode, "input_dtype": "bf16" if cfg.dtype else "f32",
                   "global_batch": cfg.T, "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "gpu_event_us": round(res["gpu_ms_per_step"] * 1e3, 2),
        "effective_tops": round(ops_total / (lat_us * 1e-6) / 1e12, 1),
        "layer_roofline_frac": round(ideal_total / lat_us, 4),
        "acbp_us": round(res["acbp_us"], 2),
        "latency_us": res["latency_us"],
        "kernels_us": {k: round(v, 2) for k, v in res["kernels_us"].items()},
        "kernels_event_us": {k: round(v, 2) for k, v in res["kernels_event_us"].items()},
        "event_overhead_us": round(res["event_overhead_us"], 2),
        "rotating_sets": res["nsets"],
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
