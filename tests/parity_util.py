"""Shared helpers of the GPU parity tests: run the GPU library and the CPU
oracle on the same seeded inputs and compare element by element.

Bar: quantized codes, scales and INT32 accumulators bit-exact (those of the
one GEMM launch the backward runs, and those of the single-GEMM launches of the
step-mask entry point); fp32 g_x and g_w within a relative Frobenius error of
1e-5, and element by element within ELEM_TOL relative error.

Why ELEM_TOL = 1e-6: the accumulators and scales are bit-exact, so the only
difference is the epilogue's rounding.  The oracle rounds acc * s_a * s_b / n
(/ T) once from fp64; the kernels form fl(fl(fl(acc) * fl(s_a * alpha)) * s_b)
with alpha = fl(1/n) exact for n a power of two (or fl(1/(n T)) for MEAN):
at most five fp32 roundings, each within 2^-24 relative, plus the oracle's
own, about 3.6e-7 in all.  Outputs whose reference is below 1e-30 (products
of denormal scales) are compared by absolute difference instead.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle as o
from hadamard_rank_linear_amd import workloads as wl

FRO_TOL = 1e-5
ELEM_TOL = 1e-6
TINY = 1e-30


def host_f32(arr, dtype):
    return arr if dtype == wl.F32 else o.bf16_bits_to_f32(arr)


def to_device(arr, dtype):
    import torch
    if dtype == wl.F32:
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()


def _fp6_e2m3_table() -> np.ndarray:
    """Value of each 6-bit FP6 E2M3 field (bit 5 sign, bits 4-3 exponent with
    bias 1, bits 2-0 mantissa; exponent 0 is subnormal, mantissa / 8)."""
    t = np.empty(64, np.float64)
    for f in range(64):
        s, e, m = f >> 5, (f >> 3) & 3, f & 7
        mag = m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 8.0)
        t[f] = -mag if s else mag
    return t


FP6_E2M3 = _fp6_e2m3_table()


def unplane(flat: np.ndarray, rows: int, pitch: int, unit: int) -> np.ndarray:
    """Row-major [rows][pitch] copy of an operand stored in K planes of
    `unit` bytes (include/hlq.h: byte k of row m at (k // unit) * rows * unit
    + m * unit + k % unit; 96 for the FP6 codes, 64 for the INT8 codes)."""
    assert pitch % unit == 0 and flat.size >= rows * pitch
    planes = flat[: rows * pitch].reshape(pitch // unit, rows, unit)
    return np.ascontiguousarray(planes.transpose(1, 0, 2)).reshape(rows, pitch)


def decode_fp6_groups(b: np.ndarray) -> np.ndarray:
    """uint8 [.., 96 * G] -> int8 [.., 128 * G]: INT4 codes stored as FP6 E2M3
    in groups of 128 (96 bytes).  Quarter Q of a group (codes 32Q .. 32Q+31)
    is a 24-byte little-endian stream, code j at bits 6j .. 6j+5; the
    quarters are stored in the order 0, 2, 1, 3.  Every field must be an
    integer in [-7, 7] and never a negative zero."""
    assert b.shape[-1] % 96 == 0
    lead = b.shape[:-1]
    g = b.reshape(lead + (b.shape[-1] // 96, 4, 24))
    out = np.empty(lead + (b.shape[-1] // 96, 4, 32), np.int8)
    for pos, q in enumerate((0, 2, 1, 3)):
        chunk = g[..., pos, :].astype(np.uint64)
        # 24 bytes = three little-endian 64-bit words
        words = [sum(chunk[..., 8 * w + k] << np.uint64(8 * k) for k in range(8)) for w in range(3)]
        for j in range(32):
            bit = 6 * j
            w, o = bit // 64, bit % 64
            f = (words[w] >> np.uint64(o)) & np.uint64(63)
            if o > 58:
                f |= (words[w + 1] << np.uint64(64 - o)) & np.uint64(63)
            f = f.astype(np.int64)
            assert not (f == 32).any(), "negative-zero FP6 field"
            v = FP6_E2M3[f]
            assert np.array_equal(v, np.round(v)) and np.abs(v).max(initial=0) <= 7, \
                "FP6 field is not an INT4 code"
            out[..., q, j] = v.astype(np.int8)
    return out.reshape(lead + (b.shape[-1] // 96 * 128,))


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """uint8 [.., K/2] -> int8 [.., K]: element 2k = low nibble, 2k+1 = high."""
    b = b.astype(np.int16)
    lo = ((b & 0xF) ^ 8) - 8
    hi = ((b >> 4) ^ 8) - 8
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


@dataclasses.dataclass
class GpuRun:
    codes: np.ndarray
    scales: np.ndarray
    g_x: np.ndarray
    g_w: np.ndarray
    inter: dict


def run_gpu(cfg, inp, x_codes=None, x_scales=None, want_acc=True, reduction=None):
    """ACBP + backward on the GPU.  When x_codes/x_scales are given (host
    arrays) the backward consumes them instead of the GPU's own ACBP output."""
    import torch
    import hadamard_rank_linear_amd as h
    gy = to_device(inp["gy"], cfg.dtype)
    x = to_device(inp["x"], cfg.dtype)
    w = to_device(inp["w"], cfg.dtype)
    codes_d, scales_d = h.hlq_compress_act(x)
    if x_codes is not None:
        codes_in = torch.from_numpy(np.ascontiguousarray(x_codes)).cuda()
        scales_in = torch.from_numpy(np.ascontiguousarray(x_scales)).cuda()
    else:
        codes_in, scales_in = codes_d, scales_d
    T, O = cfg.T, cfg.O
    I = cfg.I
    red = cfg.reduction if reduction is None else reduction
    ws_bytes = h.hlq_linear_backward_workspace_size(T, I, O, cfg.block, cfg.rank)
    ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device="cuda")
    g_x, g_w = h.hlq_linear_backward(gy, codes_in, scales_in, w, cfg.block, cfg.rank,
                                     cfg.gx_mode, cfg.gw_mode, red, workspace=ws)
    inter = {}
    if want_acc:
        # the backward's own GEMM launch, INT32 epilogue
        inter["acc_x"], inter["acc_w"] = h.hlq_gemm_pair_acc(ws, T, I, O, cfg.block, cfg.rank)
        # the single-GEMM launches of the step-mask entry point
        inter["acc_x1"] = h.hlq_gemm_gx_acc(ws, T, I, O, cfg.block, cfg.rank)
        inter["acc_w1"] = h.hlq_gemm_gw_acc(ws, T, I, O, cfg.block, cfg.rank)
    torch.cuda.synchronize()
    lay = h.hlq_workspace_layout_query(T, I, O, cfg.block, cfg.rank)
    wsh = ws.cpu().numpy()
    kxb, kwb, tl = lay["kx_pitch"], lay["kw_pitch"], lay["t_low"]

    def region(off, count, dt):
        return wsh[off: off + count * np.dtype(dt).itemsize].view(dt)

    n_gx = T if cfg.gx_mode == wl.PER_TOKEN else 1
    n_w = I if cfg.gx_mode == wl.PER_TOKEN else 1
    n_gyl = O if cfg.gw_mode == wl.PER_TOKEN else 1
    n_xl = I if cfg.gw_mode == wl.PER_TOKEN else 1
    inter.update(
        q_gy_packed=unplane(region(lay["q_gy"], T * kxb, np.uint8), T, kxb, 96),
        s_gy=region(lay["s_gy"], n_gx, np.float32).copy(),
        q_w_packed=unplane(region(lay["q_w"], I * kxb, np.uint8), I, kxb, 96),
        s_w=region(lay["s_w"], n_w, np.float32).copy(),
        q_gyl_stored=unplane(region(lay["q_gyl"], O * kwb, np.int8), O, kwb, 64),
        s_gyl=region(lay["s_gyl"], n_gyl, np.float32).copy(),
        q_xl_stored=unplane(region(lay["q_xl"], I * kwb, np.int8), I, kwb, 64),
        s_xl=region(lay["s_xl"], n_xl, np.float32).copy(),
        kxb=kxb, kwb=kwb, t_low=tl,
    )
    if want_acc:
        for k in ("acc_x", "acc_w", "acc_x1", "acc_w1"):
            inter[k] = inter[k].cpu().numpy()
    return GpuRun(codes_d.cpu().numpy(), scales_d.cpu().numpy(), g_x.cpu().numpy(),
                  g_w.cpu().numpy(), inter)


def run_oracle(cfg, inp, reduction=None):
    x = host_f32(inp["x"], cfg.dtype)
    codes, scales = o.acbp_pack(x)
    red = cfg.reduction if reduction is None else reduction
    out = o.linear_backward(host_f32(inp["gy"], cfg.dtype), codes, scales,
                            host_f32(inp["w"], cfg.dtype), cfg.block, cfg.rank,
                            cfg.gx_mode, cfg.gw_mode, red)
    return codes, scales, out


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def compare(cfg, gpu: GpuRun, ocodes, oscales, ref: dict, check_acc=True):
    """Assert the bar; returns the two relative Frobenius errors."""
    O = cfg.O
    it = gpu.inter
    # ACBP bytes and scales
    assert np.array_equal(gpu.codes, ocodes), "ACBP codes differ"
    assert np.array_equal(bits(gpu.scales), bits(oscales)), "ACBP scales differ"
    # g_x operands
    q_gy = decode_fp6_groups(it["q_gy_packed"])
    assert np.array_equal(q_gy[:, :O], ref["q_gy"]), "INT4 codes of H.g_y differ"
    assert not q_gy[:, O:].any(), "K padding of q_gy is not zero"
    assert np.array_equal(bits(it["s_gy"]), bits(ref["s_gy"])), "scales of H.g_y differ"
    q_w = decode_fp6_groups(it["q_w_packed"])
    assert np.array_equal(q_w[:, :O].T, ref["q_w"]), "INT4 codes of H.w differ"
    assert not q_w[:, O:].any(), "K padding of q_w is not zero"
    assert np.array_equal(bits(it["s_w"]), bits(ref["s_w"])), "scales of H.w differ"
    # g_w operands
    tl = it["t_low"]
    assert np.array_equal(it["q_gyl_stored"][:, :tl].T, ref["q_gyl"]), "INT8 codes of low-rank g_y differ"
    assert not it["q_gyl_stored"][:, tl:].any(), "K padding of q_gyl is not zero"
    assert np.array_equal(bits(it["s_gyl"]), bits(ref["s_gyl"])), "scales of low-rank g_y differ"
    assert np.array_equal(it["q_xl_stored"][:, :tl].T, ref["q_xl"]), "INT8 codes of low-rank x differ"
    assert not it["q_xl_stored"][:, tl:].any(), "K padding of q_xl is not zero"
    assert np.array_equal(bits(it["s_xl"]), bits(ref["s_xl"])), "scales of low-rank x differ"
    # INT32 accumulators
    if check_acc:
        assert np.array_equal(it["acc_x"].astype(np.int64), ref["acc_x"]), \
            "acc_x of the paired GEMM launch differs"
        assert np.array_equal(it["acc_w"].astype(np.int64), ref["acc_w"]), \
            "acc_w of the paired GEMM launch differs"
        assert np.array_equal(it["acc_x1"].astype(np.int64), ref["acc_x"]), \
            "acc_x of the single g_x GEMM launch differs"
        assert np.array_equal(it["acc_w1"].astype(np.int64), ref["acc_w"]), \
            "acc_w of the single g_w GEMM launch differs"
    # fp32 outputs
    assert np.isfinite(gpu.g_x).all() and np.isfinite(gpu.g_w).all()
    ex = o.rel_fro(gpu.g_x, ref["g_x"])
    ew = o.rel_fro(gpu.g_w, ref["g_w"])
    assert ex <= FRO_TOL, f"g_x relative Frobenius error {ex:.3e} > {FRO_TOL}"
    assert ew <= FRO_TOL, f"g_w relative Frobenius error {ew:.3e} > {FRO_TOL}"
    mx = o.max_rel_err(gpu.g_x, ref["g_x"], TINY)
    mw = o.max_rel_err(gpu.g_w, ref["g_w"], TINY)
    assert mx <= ELEM_TOL, f"g_x element-wise relative error {mx:.3e} > {ELEM_TOL}"
    assert mw <= ELEM_TOL, f"g_w element-wise relative error {mw:.3e} > {ELEM_TOL}"
    return ex, ew
