"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the mistake it is meant to catch.  Sources are the pages the
oracle follows: "HLQ: Fast and Efficient Backpropagation via Hadamard Low-rank
Quantization" (TL;DR; section "Hadamard Transform"; Figure 2 caption) and
"HOT: Hadamard-based Optimized Training" (scime.ai summary, "Approach").
"""
import json
import os

import numpy as np
import pytest

import oracle as o
from hadamard_rank_linear_amd import workloads as wl

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))
NS = [2, 4, 8, 16, 32, 64, 128]


def kron_hadamard(n):
    """Textbook Sylvester recursion H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# ---------------------------------------------------------------- Hadamard

@pytest.mark.parametrize("n", NS)
def test_hadamard_matches_kronecker_recursion(n):
    # catches a wrong sign/index in the popcount formula
    assert np.array_equal(o.sylvester_hadamard(n), kron_hadamard(n))


@pytest.mark.parametrize("n", NS)
def test_hadamard_orthogonal_symmetric(n):
    h = o.sylvester_hadamard(n)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))
    assert np.array_equal(h, h.T)


@pytest.mark.parametrize("n", NS)
@pytest.mark.parametrize("axis", [0, 1])
def test_fwht_equals_explicit_matrix_on_integers(n, axis):
    # integer inputs |v| <= 50: every fp32 partial sum is exact, so bit-equal
    rng = np.random.default_rng(n * 7 + axis)
    blocks, other = 3, 5
    shape = (blocks * n, other) if axis == 0 else (other, blocks * n)
    v = rng.integers(-50, 51, shape).astype(np.float32)
    got = o.fwht_blocks(v, n, axis)
    h = kron_hadamard(n).astype(np.float64)
    vb = np.moveaxis(v.astype(np.float64), axis, 0).reshape(blocks, n, other)
    ref = np.einsum("jk,bkc->bjc", h, vb).reshape(blocks * n, other)
    ref = np.moveaxis(ref, 0, axis)
    assert got.dtype == np.float32
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("n", NS)
def test_fwht_involution_on_integers(n):
    v = np.random.default_rng(n).integers(-20, 21, (4 * n,)).astype(np.float32)
    assert np.array_equal(o.fwht_blocks(o.fwht_blocks(v, n, 0), n, 0), n * v)


def test_fwht_golden_integer():
    for key in ("fwht4_integer", "fwht8_integer"):
        g = GOLDEN[key]
        got = o.fwht_blocks(np.array(g["input"], np.float32), g["n"], 0)
        assert got.tolist() == g["output"], key


def test_fwht_golden_fp32_stage_order():
    # catches descending (or any other) stage order in the fp32 butterflies
    g = GOLDEN["fwht4_fp32_stage_order"]
    v = np.array(g["input"], np.float32)
    assert v[1] == np.float32(2.0 ** -24)
    got = o.fwht_blocks(v, 4, 0)
    assert [float(x) for x in got] == g["output"]


def test_fwht_rejects_ragged_dimension():
    with pytest.raises(ValueError):
        o.fwht_blocks(np.zeros(24, np.float32), 16, 0)


# ---------------------------------------------------------------- low rank

@pytest.mark.parametrize("n", NS)
def test_lowrank_rows_are_lowest_sequency(n):
    # brute-force sign-change count on the explicit matrix
    seq = o.sequency(kron_hadamard(n))
    assert sorted(seq.tolist()) == list(range(n))     # each sequency once
    r = 1
    while r <= n:
        lowest = set(np.argsort(seq, kind="stable")[:r].tolist())
        assert lowest == set(o.lowrank_rows(n, r).tolist()), (n, r)
        r *= 2


def test_lowrank_golden():
    g = GOLDEN["lowrank_n4_r2"]
    got = o.lowrank_transform(np.array(g["input"], np.float32), g["n"], g["r"], 0)
    assert got.tolist() == g["output"]


@pytest.mark.parametrize("n,r", [(16, 8), (32, 8), (64, 16), (16, 4), (16, 1), (16, 16), (128, 32)])
def test_lowrank_is_group_average_projector(n, r):
    # (1/n) H_low^T H_low = averaging over groups of n/r consecutive tokens
    rng = np.random.default_rng(n + r)
    T, C = 4 * n, 6
    gy = rng.standard_normal((T, C))
    x = rng.standard_normal((T, C))
    got = o.lowrank_transform(gy, n, r, 0).T @ o.lowrank_transform(x, n, r, 0) / n
    g = n // r

    def avg(v):
        m = v.reshape(T // g, g, C).mean(axis=1, keepdims=True)
        return np.broadcast_to(m, (T // g, g, C)).reshape(T, C)

    ref = avg(gy).T @ avg(x)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,r", [(16, 8), (32, 8), (64, 16), (16, 4), (128, 1), (16, 16)])
def test_lowrank_pruned_form_bit_equal(n, r):
    # group sums in adjacent-pair tree order, then a size-r transform, give the
    # same fp32 bits as the full transform followed by row selection
    rng = np.random.default_rng(3 * n + r)
    T, C = 3 * n, 40
    v = (rng.standard_normal((T, C)) * np.exp(rng.standard_normal((T, C)) * 3)).astype(np.float32)
    g = n // r
    s = v.reshape(T // g, g, C)
    while s.shape[1] > 1:
        s = (s[:, 0::2] + s[:, 1::2]).astype(np.float32)
    sums = s.reshape(T // g, C)
    pruned = o.fwht_blocks(sums, r, 0)
    assert np.array_equal(pruned.view(np.uint32), o.lowrank_transform(v, n, r, 0).view(np.uint32))


# ---------------------------------------------------------------- quantizer

def test_quant_golden():
    for key in ("quant_int4_ties", "quant_int8_power_of_two", "quant_zero_group"):
        g = GOLDEN[key]
        q, s = o.quantize(np.array(g["input"], np.float32), g["qmax"], None)
        assert q.tolist() == g["codes"], key
        assert float(s[0]) == g["scale"], key


def _brute_quant(v, qmax):
    """Per-element quantizer with Python floats rounded through float32."""
    a = max(abs(float(t)) for t in v)
    if a == 0:
        return [0] * len(v), 0.0
    inv = float(np.float32(qmax) / np.float32(a))
    out = []
    for t in v:
        p = float(np.float32(float(t) * inv))     # exact product rounded once
        q = round(p)                              # Python round: half to even
        out.append(max(-qmax, min(qmax, q)))
    return out, float(np.float32(a) / np.float32(qmax))


@pytest.mark.parametrize("qmax", [7, 127])
def test_quant_matches_brute_force(qmax):
    rng = np.random.default_rng(qmax)
    v = (rng.standard_normal((6, 33)) * 3).astype(np.float32)
    v[2] = 0.0
    q, s = o.quantize(v, qmax, 1)
    for row in range(v.shape[0]):
        bq, bs = _brute_quant(v[row], qmax)
        assert q[row].tolist() == bq
        assert float(s[row]) == bs


@pytest.mark.parametrize("qmax", [7, 127])
def test_quant_invariants(qmax):
    rng = np.random.default_rng(10 + qmax)
    v = (rng.standard_t(3, (50, 64)) * 0.01).astype(np.float32)
    q, s = o.quantize(v, qmax, 1)
    assert np.abs(q).max() <= qmax
    assert (np.abs(q).max(axis=1) == qmax).all()          # per-group max hits qmax
    qn, sn = o.quantize(-v, qmax, 1)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)  # sign symmetry
    q8, s8 = o.quantize(v * np.float32(8.0), qmax, 1)      # power-of-two scaling
    assert np.array_equal(q8, q) and np.array_equal(s8, s * np.float32(8.0))
    err = np.abs(v.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert (err <= s[:, None] * (0.5 + 1e-5)).all()


@pytest.mark.parametrize("qmax", [7, 127])
def test_quant_reciprocal_overflow_group(qmax):
    # reading R5's corner: qmax / a overflows fp32 for a deep in the denormal
    # range; codes are 0 and the scale is still a / qmax
    v = np.zeros((2, 8), np.float32)
    v[0, :3] = [1e-44, -3e-45, 7e-45]
    v[1, :2] = [1.0, -0.5]
    q, s = o.quantize(v, qmax, 1)
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(qmax) / np.float32(1e-44))
    assert (q[0] == 0).all() and float(s[0]) == float(np.float32(1e-44) / np.float32(qmax))
    assert q[1, 0] == qmax and q[1, 1] == -int(np.rint(qmax / 2))


@pytest.mark.parametrize("qmax", [7, 127])
def test_quant_product_never_exceeds_qmax(qmax):
    # |fl(v * fl(qmax / a))| <= qmax(1 + 2^-24) rounds to at most qmax, so the
    # clamp of R5 never changes a code; probe groups whose absmax sweeps many
    # binades and mantissas
    rng = np.random.default_rng(77 + qmax)
    a = (rng.uniform(1, 2, 4096) * 2.0 ** rng.integers(-120, 120, 4096)).astype(np.float32)
    inv = (np.float32(qmax) / a).astype(np.float32)
    assert np.isfinite(inv).all()
    prod = (a * inv).astype(np.float32)
    assert (np.rint(prod) <= qmax).all() and (np.rint(-prod) >= -qmax).all()


def test_quant_group_axis():
    # catches a swapped scale-group axis: per-column groups along axis 0
    rng = np.random.default_rng(5)
    v = rng.standard_normal((40, 7)).astype(np.float32)
    v[:, 3] *= 100
    q, s = o.quantize(v, 7, 0)
    assert s.shape == (7,)
    assert (np.abs(q).max(axis=0) == 7).all()
    np.testing.assert_array_equal(s, (np.abs(v).max(axis=0) / np.float32(7)).astype(np.float32))


# ---------------------------------------------------------------- ACBP

def test_acbp_pack_golden():
    g = GOLDEN["acbp_pack_bytes"]
    assert o.pack_int4(np.array(g["codes"])).tolist() == g["bytes"]
    assert o.unpack_int4(np.array(g["bytes"], np.uint8)).tolist() == g["codes"]


def test_int4_pack_roundtrip_all_pairs():
    a, b = np.meshgrid(np.arange(-7, 8), np.arange(-7, 8))
    q = np.stack([a.ravel(), b.ravel()], axis=1).reshape(1, -1)
    assert np.array_equal(o.unpack_int4(o.pack_int4(q)), q.astype(np.int8))


def test_acbp_roundtrip_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    x[3] = 0.0
    codes, s = o.acbp_pack(x)
    assert codes.shape == (16, 32) and s.shape == (16,)
    xd = o.acbp_unpack(codes, s)
    assert (np.abs(xd - x) <= s[:, None] * 0.5 * (1 + 1e-5)).all()
    assert (xd[3] == 0).all() and s[3] == 0


# ---------------------------------------------------------------- integer GEMM

def test_int_matmul_brute_force():
    # non-square, so a transposed operand cannot pass
    rng = np.random.default_rng(2)
    a = rng.integers(-127, 128, (5, 9))
    b = rng.integers(-127, 128, (9, 4))
    ref = [[sum(int(a[i, k]) * int(b[k, j]) for k in range(9)) for j in range(4)] for i in range(5)]
    assert o.int_matmul(a, b).tolist() == ref


def test_int_matmul_large_exact():
    # extreme magnitudes over a long K still exact
    K = 70000
    a = np.full((2, K), 127, np.int64)
    b = np.full((K, 3), -127, np.int64)
    b[::2] = 127
    got = o.int_matmul(a, b)
    ref = 127 * 127 * (K // 2) - 127 * 127 * (K // 2)
    assert (got == ref).all()
    a[1, 0] = -127
    assert o.int_matmul(a, b)[1, 0] == ref - 2 * 127 * 127


# ---------------------------------------------------------------- whole path

@pytest.mark.parametrize("n", [16, 32, 64])
def test_exact_recovery_quant_off_full_rank(n):
    # H^T H = n I: with rank == block and no quantizer the products come back
    rng = np.random.default_rng(n)
    T, I, O = 2 * n, 12, 2 * n
    gy = rng.standard_normal((T, O))
    x = rng.standard_normal((T, I))
    w = rng.standard_normal((O, I))
    for red, div in ((o.SUM, 1.0), (o.MEAN, T)):
        out = o.linear_backward_unquantized(gy, x, w, n, n, reduction=red)
        np.testing.assert_allclose(out["g_x"], gy @ w, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out["g_w"], gy.T @ x / div, rtol=1e-12, atol=1e-12)


def test_exact_recovery_integer_inputs_bit_equal():
    rng = np.random.default_rng(9)
    n, T, I, O = 16, 32, 8, 32
    gy = rng.integers(-9, 10, (T, O)).astype(np.float64)
    x = rng.integers(-9, 10, (T, I)).astype(np.float64)
    w = rng.integers(-9, 10, (O, I)).astype(np.float64)
    out = o.linear_backward_unquantized(gy, x, w, n, n)
    assert np.array_equal(out["g_x"], gy @ w)
    assert np.array_equal(out["g_w"], gy.T @ x)


def test_golden_gw_projector():
    g = GOLDEN["gw_lowrank_projector"]
    gy = np.array(g["gy"], np.float64)[:, None]
    x = np.array(g["x"], np.float64)[:, None]
    w = np.ones((4, 1))
    out = o.linear_backward_unquantized(gy * np.ones((1, 4)), x, w, g["n"], g["r"])
    assert out["g_w"][0, 0] == g["g_w"]


def _small_case(seed=0, T=64, I=32, O=48, n=16):
    rng = np.random.default_rng(seed)
    gy = rng.standard_normal((T, O)).astype(np.float32)
    x = rng.standard_normal((T, I)).astype(np.float32)
    w = (0.02 * rng.standard_normal((O, I))).astype(np.float32)
    return gy, x, w


def test_quantized_path_codes_follow_explicit_matrix():
    # each intermediate recomputed from the explicit Hadamard matrix in fp64 and
    # the brute-force quantizer; integer-valued inputs keep fp32 sums exact
    rng = np.random.default_rng(4)
    n, r, T, I, O = 16, 4, 64, 10, 32
    gy = rng.integers(-30, 31, (T, O)).astype(np.float32)
    w = rng.integers(-30, 31, (O, I)).astype(np.float32)
    xq = rng.integers(-7, 8, (T, I))
    x_codes = o.pack_int4(xq)
    x_scales = np.ones(T, np.float32)
    out = o.linear_backward(gy, x_codes, x_scales, w, n, r, o.PER_TOKEN, o.PER_TOKEN)
    H = kron_hadamard(n)
    gy_h = np.concatenate([gy[:, b:b + n] @ H.T for b in range(0, O, n)], axis=1)
    w_h = np.concatenate([H @ w[b:b + n] for b in range(0, O, n)], axis=0)
    for t in range(T):
        bq, bs = _brute_quant(gy_h[t].astype(np.float32), 7)
        assert out["q_gy"][t].tolist() == bq and float(out["s_gy"][t]) == bs
    for i in range(I):
        bq, bs = _brute_quant(w_h[:, i].astype(np.float32), 7)
        assert out["q_w"][:, i].tolist() == bq and float(out["s_w"][i]) == bs
    Hl = H[o.lowrank_rows(n, r)]
    gyl = np.concatenate([Hl @ gy[b:b + n] for b in range(0, T, n)], axis=0)
    xl = np.concatenate([Hl @ xq[b:b + n] for b in range(0, T, n)], axis=0)
    for c in range(O):
        bq, bs = _brute_quant(gyl[:, c].astype(np.float32), 127)
        assert out["q_gyl"][:, c].tolist() == bq and float(out["s_gyl"][c]) == bs
    for c in range(I):
        bq, bs = _brute_quant(xl[:, c].astype(np.float32), 127)
        assert out["q_xl"][:, c].tolist() == bq and float(out["s_xl"][c]) == bs
    # integer GEMMs by brute force, and the fp64 epilogue
    qa, qb = out["q_gy"].astype(np.int64), out["q_w"].astype(np.int64)
    for t in (0, 17, 63):
        for i in (0, 9):
            acc = sum(int(qa[t, k]) * int(qb[k, i]) for k in range(O))
            assert out["acc_x"][t, i] == acc
            ref = np.float32(acc * float(out["s_gy"][t]) * float(out["s_w"][i]) / n)
            assert out["g_x"][t, i] == ref
    qa, qb = out["q_gyl"].astype(np.int64), out["q_xl"].astype(np.int64)
    Tl = T * r // n
    for c in (0, 31):
        for i in (0, 5):
            acc = sum(int(qa[k, c]) * int(qb[k, i]) for k in range(Tl))
            assert out["acc_w"][c, i] == acc
            ref = np.float32(acc * float(out["s_gyl"][c]) * float(out["s_xl"][i]) / n)
            assert out["g_w"][c, i] == ref


def test_per_tensor_equals_per_token_when_absmax_shared():
    # if every group has the same absmax, per-tensor and per-token coincide;
    # catches a per-tensor path that scales by the wrong maximum
    rng = np.random.default_rng(1)
    n, T, I, O = 16, 64, 32, 48
    z = rng.integers(-8, 9, (T, O)).astype(np.float32)
    z[:, 5] = 9.0                                   # every row's absmax is 9
    gy = (o.fwht_blocks(z, n, 1) / np.float32(n)).astype(np.float32)   # dyadic, exact
    assert np.array_equal(o.fwht_blocks(gy, n, 1), z)
    _, x, w = _small_case(1, T=T, I=I, O=O)
    codes, s = o.acbp_pack(x)
    a1 = o.linear_backward(gy, codes, s, w, n, 8, o.PER_TOKEN, o.PER_TOKEN)
    a2 = o.linear_backward(gy, codes, s, w, n, 8, o.PER_TENSOR, o.PER_TOKEN)
    assert a2["s_gy"].shape == (1,)
    assert np.array_equal(a1["q_gy"], a2["q_gy"])
    assert (a1["s_gy"] == a2["s_gy"][0]).all()
    # the per-tensor scale of H.w is the largest per-column one (fl(a / 7) is
    # monotone in a), and its codes are the brute-force quantizer's with it
    assert a2["s_w"].shape == (1,) and a2["s_w"][0] == a1["s_w"].max()
    w_h = o.fwht_blocks(w, n, 0)
    bq, bs = _brute_quant(w_h.ravel(), 7)
    assert np.array_equal(a2["q_w"].ravel(), np.array(bq)) and float(a2["s_w"][0]) == bs


def test_quantized_close_to_exact_product():
    # sanity: the approximation tracks the exact products at the expected scale
    gy, x, w = _small_case(2, T=256, I=64, O=64)
    codes, s = o.acbp_pack(x)
    out = o.linear_backward(gy, codes, s, w, 16, 16, o.PER_TOKEN, o.PER_TOKEN)
    xd = o.acbp_unpack(codes, s).astype(np.float64)
    assert o.rel_fro(out["g_x"], gy.astype(np.float64) @ w) < 0.25
    assert o.rel_fro(out["g_w"], gy.astype(np.float64).T @ xd) < 0.05


def test_mean_reduction_divides_gw_by_T():
    gy, x, w = _small_case(3)
    codes, s = o.acbp_pack(x)
    a = o.linear_backward(gy, codes, s, w, 16, 8, o.PER_TOKEN, o.PER_TOKEN, o.SUM)
    b = o.linear_backward(gy, codes, s, w, 16, 8, o.PER_TOKEN, o.PER_TOKEN, o.MEAN)
    np.testing.assert_allclose(b["g_w"], a["g_w"] / gy.shape[0], rtol=2e-7)
    assert np.array_equal(a["g_x"], b["g_x"])


def test_zero_groups_on_planted_rows():
    cfg = wl.BY_NAME["tiny"]
    inp = wl.make_inputs(cfg, plant_zero_rows=True)
    codes, s = o.acbp_pack(inp["x"])
    assert s[0] == 0 and (codes[0] == 0).all()
    out = o.linear_backward(inp["gy"], codes, s, inp["w"], cfg.block, cfg.rank)
    assert out["s_gy"][0] == 0 and (out["q_gy"][0] == 0).all()
    assert (out["g_x"][0] == 0).all()


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x7F7F, 0x0001], np.uint16)
    got = o.bf16_bits_to_f32(bits)
    assert got[0] == 1.0 and got[1] == -1.0 and got[2] == 0.0
    assert got[4] == np.float32(2.0 ** -133)
    assert wl.f32_to_bf16_bits(np.array([1.0, 1.00390625, 1.01171875], np.float32)).tolist() == [
        0x3F80, 0x3F80, 0x3F82]   # ties to even: 1+2^-8 -> 1, 1+3*2^-8 -> 1+2^-6


def test_quantized_path_per_tensor_follows_explicit_matrix():
    # both paths PER_TENSOR: every operand's codes from one scale (the
    # brute-force quantizer over the whole explicit-matrix transform), integer
    # GEMMs by brute force, the fp64 epilogue with the two tensor scales;
    # catches a per-tensor scale taken over the wrong operand or a per-token
    # scale left in one of the epilogues
    rng = np.random.default_rng(5)
    n, r, T, I, O = 16, 4, 64, 10, 32
    gy = rng.integers(-30, 31, (T, O)).astype(np.float32)
    w = rng.integers(-30, 31, (O, I)).astype(np.float32)
    xq = rng.integers(-7, 8, (T, I))
    x_codes = o.pack_int4(xq)
    x_scales = np.ones(T, np.float32)
    out = o.linear_backward(gy, x_codes, x_scales, w, n, r, o.PER_TENSOR, o.PER_TENSOR)
    H = kron_hadamard(n)
    gy_h = np.concatenate([gy[:, b:b + n] @ H.T for b in range(0, O, n)], axis=1)
    w_h = np.concatenate([H @ w[b:b + n] for b in range(0, O, n)], axis=0)
    Hl = H[o.lowrank_rows(n, r)]
    gyl = np.concatenate([Hl @ gy[b:b + n] for b in range(0, T, n)], axis=0)
    xl = np.concatenate([Hl @ xq[b:b + n] for b in range(0, T, n)], axis=0)
    for key, v, qmax in (("gy", gy_h, 7), ("w", w_h, 7), ("gyl", gyl, 127), ("xl", xl, 127)):
        bq, bs = _brute_quant(v.astype(np.float32).ravel(), qmax)
        assert out["s_" + key].shape == (1,)
        assert float(out["s_" + key][0]) == bs, key
        assert np.array_equal(out["q_" + key].ravel(), np.array(bq)), key
    sg, sw = float(out["s_gy"][0]), float(out["s_w"][0])
    sgl, sxl = float(out["s_gyl"][0]), float(out["s_xl"][0])
    Tl = T * r // n
    for t, i in ((0, 0), (17, 9), (63, 4)):
        acc = sum(int(out["q_gy"][t, k]) * int(out["q_w"][k, i]) for k in range(O))
        assert out["acc_x"][t, i] == acc
        assert out["g_x"][t, i] == np.float32(acc * sg * sw / n)
    for c, i in ((0, 0), (31, 5), (12, 9)):
        acc = sum(int(out["q_gyl"][k, c]) * int(out["q_xl"][k, i]) for k in range(Tl))
        assert out["acc_w"][c, i] == acc
        assert out["g_w"][c, i] == np.float32(acc * sgl * sxl / n)


def test_rel_fro_golden():
    g = GOLDEN["rel_fro_2x2"]
    assert o.rel_fro(np.array(g["a"]), np.array(g["b"])) == pytest.approx(g["value"], rel=1e-15)
    assert o.rel_fro(np.zeros(3), np.zeros(3)) == 0.0
    assert o.rel_fro(np.ones(3), np.zeros(3)) == float("inf")


def test_max_rel_err_golden():
    g = GOLDEN["max_rel_err"]
    assert o.max_rel_err(g["a1"], g["b1"], g["tiny1"]) == pytest.approx(g["value1"], rel=1e-15)
    assert o.max_rel_err(g["a2"], g["b2"], g["tiny2"]) == pytest.approx(g["value2"], rel=1e-15)
    assert o.max_rel_err(np.zeros(0), np.zeros(0), 1.0) == 0.0


def test_acbp_unpack_rounds_once_to_fp32():
    # a scale that is not a power of two: fl32(s * q) differs from the exact
    # product, so an unrounded (fp64) or twice-rounded decode fails
    g = GOLDEN["acbp_unpack_non_power_of_two"]
    s = np.array([int(g["scale_bits"], 16)], np.uint32).view(np.float32)
    got = o.acbp_unpack(np.array([g["bytes"]], np.uint8), s)
    assert got.dtype == np.float32 and got.shape == (1, 2)
    assert [hex(v) for v in got.view(np.uint32).ravel()] == [b.lower() for b in g["output_bits"]]
