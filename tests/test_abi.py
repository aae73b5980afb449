"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library loads, exports every function include/hlq.h declares, validates
arguments before enqueueing anything, and plans a consistent workspace.
"""
import ctypes
import os
import re

import numpy as np

import pytest

import hadamard_rank_linear_amd as h
from hadamard_rank_linear_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hlq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hlq_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert set(declared_functions()) == set(h.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(h.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(11):
        assert h.status_string(s) and h.status_string(s) != "unknown status"
    assert h.status_string(99) == "unknown status"
    assert h.version() >= 100


def _raw_backward(**kw):
    args = dict(gy=1 << 20, gy_dt=0, codes=1 << 20, scales=1 << 20, w=1 << 20, w_dt=0,
                T=64, I=40, O=48, block=16, rank=8, gx=0, gw=0, red=0,
                g_x=1 << 20, g_w=1 << 20, ws=1 << 20, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    lib = h.lib_handle()
    return lib.hlq_linear_backward(*(args[k] for k in (
        "gy", "gy_dt", "codes", "scales", "w", "w_dt", "T", "I", "O", "block", "rank",
        "gx", "gw", "red", "g_x", "g_w", "ws", "ws_bytes", "stream")))


@pytest.mark.parametrize("kw,status", [
    (dict(gy=None), 1),
    (dict(g_w=None), 1),
    (dict(T=0), 2),
    (dict(T=72), 2),                 # T not a multiple of the block
    (dict(O=40), 2),                 # O not a multiple of the block
    (dict(I=36), 2),                 # I not a multiple of 8
    (dict(block=24), 3),
    (dict(block=256), 3),
    (dict(rank=3), 4),
    (dict(rank=32), 4),              # rank above block
    (dict(rank=0), 4),
    (dict(gx=2), 5),
    (dict(red=7), 5),
    (dict(gy_dt=3), 6),
    (dict(w=(1 << 20) + 4), 7),      # misaligned
    (dict(O=342400, block=16), 8),   # 49 * O >= 2^24: FP6 sums not exact
    (dict(T=16 * 133144, rank=16), 8),
    (dict(ws=None), 9),
    (dict(ws_bytes=100), 9),
])
def test_validation_rejects_before_launch(kw, status):
    # pointers are fake host addresses: validation must refuse before any launch
    assert _raw_backward(**kw) == status


def test_compress_act_validation():
    lib = h.lib_handle()
    P = 1 << 20
    assert lib.hlq_compress_act(None, 0, 4, 8, P, P, None) == 1
    assert lib.hlq_compress_act(P, 5, 4, 8, P, P, None) == 6
    assert lib.hlq_compress_act(P, 0, 4, 12, P, P, None) == 2
    assert lib.hlq_compress_act(P, 0, 0, 8, P, P, None) == 2
    assert lib.hlq_compress_act(P + 2, 0, 4, 8, P, P, None) == 7


@pytest.mark.parametrize("cfg", wl.LAYERS, ids=[c.name for c in wl.LAYERS])
def test_workspace_layout_consistent(cfg):
    T, I, O, n, r = cfg.T, cfg.I, cfg.O, cfg.block, cfg.rank
    lay = h.hlq_workspace_layout_query(T, I, O, n, r)
    size = h.hlq_linear_backward_workspace_size(T, I, O, n, r)
    assert lay["total"] == size > 0
    assert lay["t_low"] == T * r // n
    # FP6 groups: 128 codes in 96 bytes
    assert lay["kx_pitch"] % 96 == 0 and lay["kx_pitch"] // 96 * 128 >= O > lay["kx_pitch"] // 96 * 128 - 128
    assert lay["kw_pitch"] % 64 == 0 and lay["kw_pitch"] >= lay["t_low"]
    regions = sorted([
        (lay["q_gy"], T * lay["kx_pitch"]), (lay["s_gy"], 4 * T),
        (lay["q_w"], I * lay["kx_pitch"]), (lay["s_w"], 4 * I),
        (lay["q_gyl"], O * lay["kw_pitch"]), (lay["s_gyl"], 4 * O),
        (lay["q_xl"], I * lay["kw_pitch"]), (lay["s_xl"], 4 * I)])
    for (a, la), (b, _) in zip(regions, regions[1:]):
        assert a % 256 == 0 and a + la <= b
    assert regions[-1][0] + regions[-1][1] <= size


SPLIT_SHAPES = [(c.T, c.I, c.O, c.block, c.rank) for c in wl.LAYERS] + [
    (64, 40, 48, 16, 16), (96, 72, 96, 32, 1), (256, 136, 192, 64, 8),
    (256, 64, 128, 128, 128), (384, 96, 256, 128, 32), (208, 264, 160, 16, 2),
    (64, 64, 4608, 16, 4), (1040, 520, 336, 16, 8), (16, 8, 16384, 16, 16),
    (65536, 8, 16, 16, 16), (1040, 768, 2304, 16, 8), (1056, 3072, 768, 32, 8),
    (1024, 14336, 4096, 64, 16), (2064, 2304, 256, 16, 4), (528, 768, 2304, 16, 8)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_split_k_partials_fit(shape):
    # regression: a split-K GEMM must always have its partial-sum buffer
    T, I, O, n, r = shape
    lay = h.hlq_workspace_layout_query(T, I, O, n, r)
    need = 0
    if lay["gx_splits"] > 1:
        need = max(need, lay["gx_splits"] * T * I * 4)
    if lay["gw_splits"] > 1:
        need = max(need, lay["gw_splits"] * O * I * 4)
    assert lay["partial_bytes"] >= need
    assert lay["partial"] % 256 == 0
    assert lay["partial"] + lay["partial_bytes"] <= lay["total"]
    for other in ("q_gy", "q_w", "q_gyl", "q_xl"):
        assert lay[other] < lay["partial"] or lay["partial_bytes"] == 0


def test_workspace_size_zero_for_invalid_shape():
    assert h.hlq_linear_backward_workspace_size(64, 40, 48, 24, 8) == 0
    with pytest.raises(h.HLQError):
        h.hlq_workspace_layout_query(64, 40, 40, 16, 8)


# ---------------------------------------------- layer-wise quantizer selection

def test_lqs_select_matches_oracle_rule():
    import numpy as np
    import oracle as o
    rng = np.random.default_rng(3)
    cases = [np.zeros(16)]
    for _ in range(300):
        st = rng.uniform(0, 1, 16) * (rng.uniform(0, 1, 16) < 0.9)
        st[[2, 6, 10, 14]] = st[[1, 5, 9, 13]] * rng.choice([0.5, 1.0, 1.4, 1.5, 1.6, 3.0])
        cases.append(st)
    for st in cases:
        for thr in (0.0, 0.5, 2.0):
            assert h.hlq_lqs_select(st.tolist(), thr) == o.lqs_select(st, thr)


def test_lqs_select_rejects_bad_threshold():
    with pytest.raises(h.HLQError):
        h.hlq_lqs_select([0.0] * 16, -0.1)
    with pytest.raises(h.HLQError):
        h.hlq_lqs_select([0.0] * 16, float("nan"))


def test_lqs_workspace_size():
    assert h.hlq_lqs_workspace_size(64, 40, 48, 16, 8) > 0
    assert h.hlq_lqs_workspace_size(72, 40, 48, 16, 8) == 0    # T not a multiple of 16


@pytest.mark.parametrize("kw,status", [
    (dict(gy=None), 1), (dict(stats=None), 1), (dict(T=72), 2), (dict(block=24), 3),
    (dict(rank=3), 4), (dict(gy_dt=2), 6), (dict(ws_bytes=16), 9), (dict(stats=(1 << 20) + 8), 7),
    (dict(T=1 << 20, O=4096, rank=1), 8),   # g_y of 8 GiB: beyond 32-bit offsets
])
def test_lqs_accumulate_validates_before_launch(kw, status):
    args = dict(gy=1 << 20, gy_dt=0, codes=1 << 20, scales=1 << 20, w=1 << 20, w_dt=0,
                T=64, I=40, O=48, block=16, rank=8, stats=1 << 20, ws=1 << 20,
                ws_bytes=1 << 40, stream=None)
    args.update(kw)
    lib = h.lib_handle()
    got = lib.hlq_lqs_accumulate(*(args[k] for k in (
        "gy", "gy_dt", "codes", "scales", "w", "w_dt", "T", "I", "O", "block", "rank",
        "stats", "ws", "ws_bytes", "stream")))
    assert got == status


@pytest.mark.parametrize("fn", ["hlq_gemm_pair_acc", "hlq_gemm_gx_acc", "hlq_gemm_gw_acc"])
@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), 1), (dict(acc=None), 1), (dict(T=72), 2), (dict(block=24), 3),
    (dict(rank=3), 4), (dict(ws_bytes=100), 9), (dict(acc=(1 << 20) + 4), 7),
])
def test_accumulator_exports_validate_before_launch(fn, kw, status):
    # the INT32 exports check the caller's workspace size like the backward
    args = dict(ws=1 << 20, ws_bytes=1 << 40, T=64, I=40, O=48, block=16, rank=8,
                acc=1 << 20, stream=None)
    args.update(kw)
    lib = h.lib_handle()
    head = [args[k] for k in ("ws", "ws_bytes", "T", "I", "O", "block", "rank")]
    if fn == "hlq_gemm_pair_acc":
        got = lib.hlq_gemm_pair_acc(*head, args["acc"], 1 << 21, args["stream"])
    else:
        got = getattr(lib, fn)(*head, args["acc"], args["stream"])
    assert got == status


def test_binding_checks_caller_buffers():
    # dtype / shape of caller-supplied buffers are checked before any call
    import torch
    x = torch.zeros((16, 8))
    with pytest.raises(TypeError):
        h.hlq_compress_act(x, x_codes=torch.zeros((16, 4)), x_scales=torch.zeros(16))
    with pytest.raises(ValueError):
        h.hlq_compress_act(x, x_codes=torch.zeros((16, 8), dtype=torch.uint8),
                           x_scales=torch.zeros(16))


@pytest.mark.parametrize("kw,status", [
    (dict(gy=None), 1), (dict(C=12), 2), (dict(H=9, W=9), 2),  # C % 8; N*P*Q = 162
    (dict(stride=0), 2), (dict(R=40), 2), (dict(block=24), 3), (dict(rank=3), 4),
    (dict(gx=0), 5),                                         # per-token g_x: not supported
    (dict(red=3), 5), (dict(gy_dt=4), 6), (dict(w=(1 << 20) + 8), 7),
    (dict(O=16, R=150, S=150, H=165, W=165, pad=0), 8),      # 49*O*R*S >= 2^24 (FP6 sums)
    (dict(ws_bytes=64), 9),
])
def test_conv_backward_validates_before_launch(kw, status):
    args = dict(gy=1 << 20, gy_dt=1, codes=1 << 20, scales=1 << 20, w=1 << 20, w_dt=1,
                N=2, H=8, W=8, C=16, O=32, R=3, S=3, stride=1, pad=1, block=16, rank=8,
                gx=1, gw=0, red=0, g_x=1 << 20, g_w=1 << 20, ws=1 << 20, ws_bytes=1 << 40,
                stream=None)
    args.update(kw)
    lib = h.lib_handle()
    got = lib.hlq_conv_backward(*(args[k] for k in (
        "gy", "gy_dt", "codes", "scales", "w", "w_dt", "N", "H", "W", "C", "O", "R", "S",
        "stride", "pad", "block", "rank", "gx", "gw", "red", "g_x", "g_w", "ws", "ws_bytes",
        "stream")))
    assert got == status


def test_conv_workspace_covers_the_linear_layout():
    c = wl.CONV_BY_NAME["resnet50_s3_conv3x3"]
    conv = h.hlq_conv_backward_workspace_size(c.N, c.H, c.W, c.C, c.O, c.R, c.S, c.stride, c.pad,
                                              c.block, c.rank)
    lin = h.hlq_linear_backward_workspace_size(c.T, c.I, c.O, c.block, c.rank)
    assert conv > lin > 0


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(ydt=5), 6), (dict(I=48), 2), (dict(T=0), 2),
    (dict(y=(1 << 20) + 4), 7)])
def test_forward_validates_before_launch(kw, status):
    args = dict(x=1 << 20, w=1 << 20, T=64, I=64, O=32, y=1 << 20, ydt=1, codes=1 << 20,
                scales=1 << 20, stream=None)
    args.update(kw)
    lib = h.lib_handle()
    assert lib.hlq_linear_forward(*(args[k] for k in (
        "x", "w", "T", "I", "O", "y", "ydt", "codes", "scales", "stream"))) == status


# ------------------------------------------------ FP6 storage of the g_x codes

def test_fp6_field_values_follow_e2m3():
    # E2M3: sign bit 5, exponent bits 4-3 (bias 1), mantissa bits 2-0
    from parity_util import FP6_E2M3
    fields = {0: 0b000000, 1: 0b001000, 2: 0b010000, 3: 0b010100, 4: 0b011000,
              5: 0b011010, 6: 0b011100, 7: 0b011110}
    for q, f in fields.items():
        assert FP6_E2M3[f] == q
        assert FP6_E2M3[f | 0b100000] == -q
    assert FP6_E2M3[0b000001] == 0.125 and FP6_E2M3[0b011111] == 7.5


def _encode_fp6_groups(codes):
    # plain bit-stream writer: quarter Q of each group of 128 at byte
    # 24 * pos(Q), pos = (0, 2, 1, 3)[Q], code j of a quarter at bits 6j
    enc = {q: (0b100000 if q < 0 else 0) | {0: 0, 1: 8, 2: 16, 3: 20, 4: 24, 5: 26, 6: 28, 7: 30}[abs(q)]
           for q in range(-7, 8)}
    rows, k = codes.shape
    out = np.zeros((rows, k // 128 * 96), np.uint8)
    for r in range(rows):
        for g in range(k // 128):
            for q in range(4):
                pos = (0, 2, 1, 3)[q]
                acc = 0
                for j in range(32):
                    acc |= enc[int(codes[r, 128 * g + 32 * q + j])] << (6 * j)
                out[r, 96 * g + 24 * pos: 96 * g + 24 * pos + 24] = np.frombuffer(
                    acc.to_bytes(24, "little"), np.uint8)
    return out


def test_fp6_group_decoder_round_trip_and_hand_bytes():
    from parity_util import decode_fp6_groups
    rng = np.random.default_rng(5)
    codes = rng.integers(-7, 8, size=(3, 256)).astype(np.int8)
    assert np.array_equal(decode_fp6_groups(_encode_fp6_groups(codes)), codes)
    # hand bytes: code 1 at K 0 -> field 8 in byte 0; code -7 at K 32
    # (quarter 1, stored second-to-... third: position 2) -> field 62 at byte 48;
    # code 3 at K 64 + 1 (quarter 2, position 1, bits 6-11) -> byte 24 bits 6-7
    # hold 20 & 3 = 0, byte 25 bits 0-3 hold 20 >> 2 = 5
    c = np.zeros((1, 128), np.int8)
    c[0, 0], c[0, 32], c[0, 65] = 1, -7, 3
    b = _encode_fp6_groups(c)
    assert b[0, 0] == 8 and b[0, 48] == 62 and b[0, 24] == 0 and b[0, 25] == 5
    assert int(b.sum()) == 8 + 62 + 5
    assert np.array_equal(decode_fp6_groups(b), c)


def test_k_plane_decoder_follows_the_header_formula():
    """unplane inverts the K-plane storage of include/hlq.h (byte k of row m
    at (k // U) * rows * U + m * U + k % U), checked byte by byte."""
    from parity_util import unplane
    for rows, pitch, unit in ((5, 192, 96), (3, 128, 64), (7, 64, 64)):
        flat = np.zeros(rows * pitch, np.int64)
        for m in range(rows):
            for k in range(pitch):
                flat[(k // unit) * rows * unit + m * unit + k % unit] = 1000 * m + k
        got = unplane(flat, rows, pitch, unit)
        assert got.shape == (rows, pitch)
        assert np.array_equal(got, 1000 * np.arange(rows)[:, None] + np.arange(pitch)[None, :])
