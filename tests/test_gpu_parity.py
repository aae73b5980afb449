"""GPU parity: libhlq.so (gfx950) against the CPU oracle on the same seeded inputs.

Every case prints its name before it touches the GPU.  Shapes span several
GEMM tiles with ragged M/N/K tails; the layer configs run at reduced token
counts element by element and at their full sizes (the sizes the benchmark
times).  The bar: codes, scales and INT32 accumulators bit-exact, fp32 g_x and
g_w within relative Frobenius error 1e-5.
"""
import dataclasses

import numpy as np
import pytest

import oracle as o
from hadamard_rank_linear_amd import workloads as wl
from parity_util import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def _case(cfg, plant=False, reduction=None, seed=0):
    _say(f"{cfg.name} T={cfg.T} I={cfg.I} O={cfg.O} n={cfg.block} r={cfg.rank} "
         f"modes=({cfg.gx_mode},{cfg.gw_mode}) dtype={cfg.dtype} red={reduction} "
         f"plant={plant} seed={seed}")
    inp = wl.make_inputs(cfg, seed=seed, plant_zero_rows=plant)
    ocodes, oscales, ref = run_oracle(cfg, inp, reduction=reduction)
    gpu = run_gpu(cfg, inp, x_codes=ocodes, x_scales=oscales, reduction=reduction)
    ex, ew = compare(cfg, gpu, ocodes, oscales, ref)
    _say(f"ok rel_fro g_x={ex:.2e} g_w={ew:.2e}")


# ----------------------------------------------------------------- tiny layer

def test_tiny_config_exact():
    _case(wl.BY_NAME["tiny"])


def test_tiny_mean_reduction():
    _case(wl.BY_NAME["tiny"], reduction=wl.MEAN)


@pytest.mark.parametrize("gx_mode,gw_mode", [(0, 1), (1, 0), (1, 1)])
def test_tiny_mode_combinations(gx_mode, gw_mode):
    _case(dataclasses.replace(wl.BY_NAME["tiny"], gx_mode=gx_mode, gw_mode=gw_mode))


def test_tiny_zero_groups():
    # planted all-zero token / weight row: scale 0 and codes 0 on every path
    _case(wl.BY_NAME["tiny"], plant=True)
    _case(dataclasses.replace(wl.BY_NAME["tiny"], gx_mode=1, gw_mode=1), plant=True)


def test_tiny_denormal_group():
    # token 1 of g_y holds denormals only: qmax / a overflows fp32, so that
    # token's g_x-path codes are all zero while its scale stays a / 7
    cfg = dataclasses.replace(wl.BY_NAME["tiny"], dtype=wl.F32)
    _say(f"denormal token row: {cfg.name} T={cfg.T} I={cfg.I} O={cfg.O}")
    inp = wl.make_inputs(cfg, seed=3)
    gy = inp["gy"].copy()
    gy[1, :] = (np.arange(cfg.O) % 5 - 2).astype(np.float32) * np.float32(1.4e-45)
    inp = dict(inp, gy=gy)
    ocodes, oscales, ref = run_oracle(cfg, inp)
    assert (ref["q_gy"][1] == 0).all() and ref["s_gy"][1] > 0
    gpu = run_gpu(cfg, inp, x_codes=ocodes, x_scales=oscales)
    compare(cfg, gpu, ocodes, oscales, ref)


# ----------------------------------------------- block sizes, ranks, tails

SHAPES = [
    # (T, I, O, n, r, dtype)
    (64, 40, 48, 16, 16, wl.F32),       # N tail (I=40), K=48 padded to 128
    (96, 72, 96, 32, 1, wl.BF16),       # rank 1
    (256, 136, 192, 64, 8, wl.BF16),
    (256, 64, 128, 128, 128, wl.F32),   # full rank at the largest block
    (384, 96, 256, 128, 32, wl.BF16),
    (208, 264, 160, 16, 2, wl.F32),     # M tail (T=208), N tail (264)
    (64, 64, 4608, 16, 4, wl.BF16),     # rows longer than the register buffer
    (1040, 520, 336, 16, 8, wl.BF16),   # several tiles, ragged everywhere
]


@pytest.mark.parametrize("T,I,O,n,r,dt", SHAPES)
@pytest.mark.parametrize("gx_mode,gw_mode", [(0, 0), (1, 1)])
def test_shapes(T, I, O, n, r, dt, gx_mode, gw_mode):
    base = wl.BY_NAME["vitb_qkv"] if dt == wl.BF16 else wl.BY_NAME["tiny"]
    cfg = dataclasses.replace(base, T=T, I=I, O=O, block=n, rank=r, dtype=dt,
                              gx_mode=gx_mode, gw_mode=gw_mode, index=100 + T % 97)
    _case(cfg)


# The g_w tiles of the pair launch split K over 2, 3 and 4 workgroups when
# T' is long against the rest of the launch (the last to arrive adds the
# others' INT32 sums): the accumulators stay bit-exact for every split count.
SPLIT_SHAPES = [
    # (T, I, O, n, r, dtype): g_w tiles x K splits
    (2048, 128, 64, 16, 8, wl.F32),     # 1 tile x 2 splits of 4 stages
    (3072, 520, 336, 16, 8, wl.BF16),   # 30 tiles (ragged O and I) x 3 splits
    (2048, 384, 256, 16, 16, wl.BF16),  # 12 tiles x 4 splits
]


@pytest.mark.parametrize("T,I,O,n,r,dt", SPLIT_SHAPES)
@pytest.mark.parametrize("gx_mode,gw_mode", [(0, 0), (1, 1)])
def test_split_k_shapes(T, I, O, n, r, dt, gx_mode, gw_mode):
    base = wl.BY_NAME["vitb_qkv"] if dt == wl.BF16 else wl.BY_NAME["tiny"]
    cfg = dataclasses.replace(base, T=T, I=I, O=O, block=n, rank=r, dtype=dt,
                              gx_mode=gx_mode, gw_mode=gw_mode, index=200 + T % 89)
    _case(cfg)


# Long-K grids that 128 x 128 tiles would run in many rounds take 256 x 256
# tiles (512-thread workgroups); this one is ragged along every dimension
# (T, I past the last tile, O past the last 128-value FP6 group).
def test_large_tile_pair_ragged():
    base = wl.BY_NAME["vitb_qkv"]
    cfg = dataclasses.replace(base, T=1040, I=13000, O=4112, block=16, rank=8, dtype=wl.BF16,
                              gx_mode=0, gw_mode=0, index=311)
    _case(cfg)


# Accumulators at their exactness limits.  Inputs planted so that every
# transformed value of an operand has the same magnitude (a one-hot first
# element per Hadamard block transforms to a block of ones), hence every
# code is qmax and every accumulator the largest the API admits.
def _limit_case(T, I, O, n, r, gy, x, w, expect_x=None, expect_w=None):
    base = wl.BY_NAME["tiny"]
    cfg = dataclasses.replace(base, T=T, I=I, O=O, block=n, rank=r, dtype=wl.F32,
                              gx_mode=0, gw_mode=0, index=401)
    _say(f"limit case T={T} I={I} O={O} n={n} r={r}")
    inp = {"gy": gy, "x": x, "w": w}
    ocodes, oscales, ref = run_oracle(cfg, inp)
    gpu = run_gpu(cfg, inp, x_codes=ocodes, x_scales=oscales)
    compare(cfg, gpu, ocodes, oscales, ref)
    if expect_x is not None:
        assert (gpu.inter["acc_x"] == expect_x).all()
    if expect_w is not None:
        assert (gpu.inter["acc_w"] == expect_w).all()


def test_gx_accumulator_at_the_fp6_exactness_limit():
    # O = 342384 (<= 342391): acc_x = 49 * O = 16776816 < 2^24, every fp32
    # partial sum of the FP6 product an exact integer up to the last one
    T, I, O, n = 16, 8, 342384, 16
    gy = np.zeros((T, O), np.float32)
    gy[:, ::n] = 1.0
    w = np.zeros((O, I), np.float32)
    w[::n, :] = 1.0
    x = np.random.default_rng(7).standard_normal((T, I)).astype(np.float32)
    _limit_case(T, I, O, n, 8, gy, x, w, expect_x=49 * O)


def test_gw_accumulator_at_the_int32_limit():
    # T' = T = 133136 (<= 133143, full rank): acc_w = 127^2 * T' = 2147350544
    # < 2^31; the g_w tile's K also splits over workgroups here
    T, I, O, n = 133136, 8, 16, 16
    gy = np.zeros((T, O), np.float32)
    gy[::n, :] = 1.0
    x = np.zeros((T, I), np.float32)
    x[::n, :] = 1.0
    w = np.random.default_rng(8).standard_normal((O, I)).astype(np.float32) * 0.02
    _limit_case(T, I, O, n, 16, gy, x, w, expect_w=127 * 127 * T)


# ----------------------------------------------- layer configs, reduced tokens

REDUCED_T = {"vitb_qkv": 1040, "vitb_fc2": 1056, "llama3_8b_down": 1024,
             "resnet50_s3_conv": 2064}
FULL_LAYERS = list(REDUCED_T)


@pytest.mark.parametrize("name", FULL_LAYERS)
def test_layer_config_reduced_tokens(name):
    cfg = wl.BY_NAME[name].with_tokens(REDUCED_T[name])
    _case(cfg)


# ----------------------------------------------- layer configs, full size

@pytest.mark.parametrize("name", FULL_LAYERS)
def test_layer_config_full_size(name):
    _case(wl.BY_NAME[name])


# ----------------------------------------------- behaviour

def test_gpu_acbp_matches_oracle_bf16_and_f32():
    for cfg in (wl.BY_NAME["tiny"], wl.BY_NAME["vitb_qkv"].with_tokens(64)):
        _say(f"acbp {cfg.name}")
        inp = wl.make_inputs(cfg, plant_zero_rows=True)
        import hadamard_rank_linear_amd as h
        from parity_util import host_f32, to_device
        codes, scales = h.hlq_compress_act(to_device(inp["x"], cfg.dtype))
        oc, os_ = o.acbp_pack(host_f32(inp["x"], cfg.dtype))
        assert np.array_equal(codes.cpu().numpy(), oc)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def test_deterministic_reruns():
    cfg = wl.BY_NAME["vitb_qkv"].with_tokens(528)
    _say("determinism")
    inp = wl.make_inputs(cfg)
    a = run_gpu(cfg, inp, want_acc=False)
    b = run_gpu(cfg, inp, want_acc=False)
    assert np.array_equal(a.g_x.view(np.uint32), b.g_x.view(np.uint32))
    assert np.array_equal(a.g_w.view(np.uint32), b.g_w.view(np.uint32))


def test_invalid_arguments_enqueue_nothing():
    import torch
    import hadamard_rank_linear_amd as h
    _say("validation")
    gy = torch.zeros((64, 48), dtype=torch.float32, device="cuda")
    w = torch.zeros((48, 40), dtype=torch.float32, device="cuda")
    codes = torch.zeros((64, 20), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((64,), dtype=torch.float32, device="cuda")
    gx = torch.full((64, 40), 7.0, device="cuda")
    gw = torch.full((48, 40), 7.0, device="cuda")
    with pytest.raises(h.HLQError):
        h.hlq_linear_backward(gy, codes, sc, w, 24, 8, g_x=gx, g_w=gw)      # bad block
    with pytest.raises(h.HLQError):
        h.hlq_linear_backward(gy, codes, sc, w, 16, 3, g_x=gx, g_w=gw)      # bad rank
    with pytest.raises(h.HLQError):
        h.hlq_linear_backward(gy, codes, sc, w, 16, 8, gx_mode=2, g_x=gx, g_w=gw)
    small = torch.zeros((16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(h.HLQError):
        h.hlq_linear_backward(gy, codes, sc, w, 16, 8, g_x=gx, g_w=gw, workspace=small)
    torch.cuda.synchronize()
    assert (gx == 7.0).all() and (gw == 7.0).all()


@pytest.mark.parametrize("I", [8, 520, 1032, 2048, 2056, 3080])
@pytest.mark.parametrize("dt", [wl.F32, wl.BF16])
def test_gpu_acbp_row_widths(I, dt):
    # every row length class of the ACBP kernel (rows kept in registers in
    # one, two or four 512-element chunks, ragged last chunk, rows read twice)
    import dataclasses
    import hadamard_rank_linear_amd as h
    from parity_util import host_f32, to_device
    cfg = dataclasses.replace(wl.BY_NAME["vitb_qkv"], T=48, I=I, dtype=dt, index=90 + I % 7)
    _say(f"acbp I={I} dtype={dt}")
    inp = wl.make_inputs(cfg, plant_zero_rows=True)
    codes, scales = h.hlq_compress_act(to_device(inp["x"], dt))
    oc, os_ = o.acbp_pack(host_f32(inp["x"], dt))
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("gy_dt,w_dt", [(wl.BF16, wl.F32), (wl.F32, wl.BF16)])
def test_mixed_input_dtypes(gy_dt, w_dt):
    # g_y and w in different element types: each input is read in its own
    # type (backward and LQS statistics)
    import dataclasses
    import torch
    import hadamard_rank_linear_amd as h
    from parity_util import host_f32, to_device
    cfg = dataclasses.replace(wl.BY_NAME["vitb_qkv"], T=320, I=200, O=192, block=32, rank=8, index=91)
    _say(f"mixed dtypes gy={gy_dt} w={w_dt}")
    inp_b = wl.make_inputs(dataclasses.replace(cfg, dtype=wl.BF16))
    inp_f = wl.make_inputs(dataclasses.replace(cfg, dtype=wl.F32))
    gy_h = inp_b["gy"] if gy_dt == wl.BF16 else inp_f["gy"]
    w_h = inp_b["w"] if w_dt == wl.BF16 else inp_f["w"]
    gy32, w32 = host_f32(gy_h, gy_dt), host_f32(w_h, w_dt)
    codes, scales = o.acbp_pack(inp_f["x"])
    ref = o.linear_backward(gy32, codes, scales, w32, cfg.block, cfg.rank,
                            cfg.gx_mode, cfg.gw_mode, cfg.reduction)
    gy, w = to_device(gy_h, gy_dt), to_device(w_h, w_dt)
    c = torch.from_numpy(codes).cuda()
    s = torch.from_numpy(scales).cuda()
    g_x, g_w = h.hlq_linear_backward(gy, c, s, w, cfg.block, cfg.rank, cfg.gx_mode,
                                     cfg.gw_mode, cfg.reduction)
    stats = h.hlq_lqs_accumulate(gy, c, s, w, cfg.block, cfg.rank)
    torch.cuda.synchronize()
    assert o.rel_fro(g_x.cpu().numpy(), ref["g_x"]) <= 1e-5
    assert o.rel_fro(g_w.cpu().numpy(), ref["g_w"]) <= 1e-5
    ost = o.lqs_stats(gy32, codes, scales, w32, cfg.block, cfg.rank)
    np.testing.assert_allclose(stats.cpu().numpy(), ost, rtol=1e-9, atol=0)


# ----------------------------------------------- exact quantizer ties

def _tie_count(v, inv):
    """Elements whose fl32(v * inv) lies exactly halfway between integers."""
    p = (np.asarray(v, np.float32) * np.asarray(inv, np.float32)).astype(np.float32)
    return int(np.count_nonzero(p - np.floor(p) == np.float32(0.5)))


def _odd_with_max(rng, shape, peak, axis):
    """Odd integers in [-(peak-1), peak-1] with one entry +-peak (even) per
    line along `axis`: the group maximum is peak, every other entry odd."""
    u = 2 * rng.integers(-(peak // 2), peak // 2, shape) + 1
    u = np.moveaxis(u, axis, -1)
    idx = rng.integers(0, u.shape[-1], u.shape[:-1])
    np.put_along_axis(u, idx[..., None], peak * rng.choice([-1, 1], u.shape[:-1])[..., None], -1)
    return np.moveaxis(u, -1, axis).astype(np.float64)


@pytest.mark.parametrize("dt,T,I,O", [(wl.F32, 64, 64, 64), (wl.BF16, 256, 128, 256)])
@pytest.mark.parametrize("gx_mode", [0, 1])
def test_quantizer_ties_gx_path(dt, T, I, O, gx_mode):
    # Transformed g_y rows and w columns are odd integers with group maximum
    # 14, so inv = fl(7 / 14) = 0.5 and every odd value lands on k + 1/2:
    # round half to even decides most INT4 codes.  g_y = H u / 16 per block
    # (multiples of 1/16 below 16, exact in bf16 and fp32), so the fp32
    # butterflies give back u exactly.
    n = 16
    rng = np.random.default_rng(21)
    H = o.sylvester_hadamard(n).astype(np.float64)
    u_gy = _odd_with_max(rng, (T, O), 14, axis=1)
    u_w = _odd_with_max(rng, (O, I), 14, axis=0)
    gy = np.concatenate([u_gy[:, b:b + n] @ H / n for b in range(0, O, n)], axis=1)
    w = np.concatenate([H @ u_w[b:b + n] / n for b in range(0, O, n)], axis=0)
    cfg = dataclasses.replace(wl.BY_NAME["tiny"], T=T, I=I, O=O, block=n, rank=8, dtype=dt,
                              gx_mode=gx_mode, gw_mode=0, index=77)
    inp = wl.make_inputs(cfg, seed=5)
    to_store = (lambda a: a.astype(np.float32)) if dt == wl.F32 else \
        (lambda a: wl.f32_to_bf16_bits(a.astype(np.float32)))
    inp = dict(inp, gy=to_store(gy), w=to_store(w))
    _say(f"quantizer ties on the g_x path dtype={dt} T={T} I={I} O={O} gx_mode={gx_mode}")
    ocodes, oscales, ref = run_oracle(cfg, inp)
    gy_h = o.fwht_blocks(gy.astype(np.float32), n, 1)
    assert np.array_equal(gy_h, u_gy.astype(np.float32))
    ties = _tie_count(gy_h, 0.5) + _tie_count(o.fwht_blocks(w.astype(np.float32), n, 0), 0.5)
    assert ties > (T * O + O * I) // 2, "the inputs should plant exact ties"
    gpu = run_gpu(cfg, inp, x_codes=ocodes, x_scales=oscales)
    compare(cfg, gpu, ocodes, oscales, ref)


def test_quantizer_ties_gw_path():
    # rank 1: the low-rank value of a block is its plain sum.  g_y block sums
    # are odd with column maximum 254 (inv = fl(127 / 254) = 0.5: every odd
    # sum is a tie); x decodes with scale 127/32 and its block code sums are
    # +-64 (low-rank value +-254, the column maximum: inv 0.5) or +-32
    # (low-rank value +-127, times 0.5 exactly +-63.5): ties again.
    n, T, I, O = 16, 128, 32, 32
    nb = T // n
    rng = np.random.default_rng(22)
    cfg = dataclasses.replace(wl.BY_NAME["tiny"], T=T, I=I, O=O, block=n, rank=1, dtype=wl.F32,
                              gx_mode=0, gw_mode=0, index=78)
    inp = wl.make_inputs(cfg, seed=6)
    sums = _odd_with_max(rng, (nb, O), 254, axis=0)
    gy = rng.integers(-20, 21, (T, O)).astype(np.float64)
    for b in range(nb):
        gy[b * n + n - 1] = sums[b] - gy[b * n:b * n + n - 1].sum(axis=0)
    q = np.zeros((T, I), np.int64)
    for i in range(I):
        targets = rng.choice([-32, 32, -32, 32, 5, -11], nb)
        targets[rng.integers(0, nb)] = 64 * rng.choice([-1, 1])
        for b in range(nb):
            left, k = int(targets[b]), b * n
            sgn = 1 if left >= 0 else -1
            while left != 0:
                step = sgn * min(7, abs(left))
                q[k, i] = step
                left -= step
                k += 1
    codes = o.pack_int4(q)
    scales = np.full(T, 127.0 / 32.0, np.float32)
    inp = dict(inp, gy=gy.astype(np.float32))
    _say(f"quantizer ties on the g_w path T={T} I={I} O={O} n={n} r=1")
    ref = o.linear_backward(inp["gy"], codes, scales, inp["w"], n, 1, 0, 0, cfg.reduction)
    gyl = o.lowrank_transform(inp["gy"], n, 1, 0)
    xl = o.lowrank_transform(o.acbp_unpack(codes, scales), n, 1, 0)
    assert np.array_equal(gyl, sums.astype(np.float32))
    assert (np.abs(xl).max(axis=0) == 254).all()
    ties = _tie_count(gyl, 0.5) + _tie_count(xl, 0.5)
    assert ties >= nb * O // 2, "the inputs should plant exact ties"
    gpu = run_gpu(cfg, inp, x_codes=codes, x_scales=scales)
    ocodes, oscales = o.acbp_pack(inp["x"])   # run_gpu also packs inp["x"]
    compare(cfg, gpu, ocodes, oscales, ref)


# ----------------------------------------------- forward with fused ACBP

@pytest.mark.parametrize("T,I,O", [(12608, 768, 2304), (1040, 3072, 768), (200, 96, 72),
                                   (64, 32, 16)])
def test_forward_with_fused_acbp(T, I, O):
    # y = x . w^T on the bf16 matrix cores against the fp64 product (fp32
    # output: within 1e-5 relative Frobenius error; bf16 output: within one
    # bf16 rounding of it), and the codes / scales the same launch emits
    # bit-identical to the oracle's ACBP of x
    import torch
    import hadamard_rank_linear_amd as h
    from parity_util import to_device
    _say(f"forward T={T} I={I} O={O}")
    cfg = dataclasses.replace(wl.BY_NAME["vitb_qkv"], T=T, I=I, O=O, index=95 + T % 5)
    inp = wl.make_inputs(cfg, plant_zero_rows=True)
    x32, w32 = o.bf16_bits_to_f32(inp["x"]), o.bf16_bits_to_f32(inp["w"])
    ref = o.linear_forward(x32, w32)
    oc, os_ = o.acbp_pack(x32)
    x, w = to_device(inp["x"], wl.BF16), to_device(inp["w"], wl.BF16)
    y, codes, scales = h.hlq_linear_forward(x, w, y_dtype=torch.float32)
    y16 = h.hlq_linear_forward(x, w, compress=False)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oc), "ACBP codes of the forward differ"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    e = o.rel_fro(y.cpu().numpy(), ref)
    assert e <= 1e-5, f"forward relative Frobenius error {e:.3e}"
    y16f = y16.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(y16f - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30 + np.abs(y.cpu().numpy() - ref) * 2)
