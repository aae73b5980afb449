"""Pins of the oracle's layer-wise quantizer selection statistics (reading R10
of the oracle header) against things other than the oracle itself: a
per-element brute force built from explicit Hadamard matrices, the per-element
error bound of an absmax quantizer, the equal-absmax invariant, a planted
outlier token, and the threshold rule on hand-made statistics.
"""
import numpy as np
import pytest

import oracle as o


def _brute_stats(gy, x_codes, x_scales, w, n, r):
    """Element-by-element statistics with explicit matrices and scalar fp32
    arithmetic.  Inputs are integer-valued (and x dyadic), so every transform
    is exact and equals the fp32 butterfly network."""
    T, O = gy.shape
    I = w.shape[1]
    H = o.sylvester_hadamard(n)
    keep = [j * (n // r) for j in range(r)]
    f32 = np.float32
    xq = o.unpack_int4(x_codes).astype(np.int64)
    x = [[float(f32(x_scales[t]) * f32(xq[t, i])) for i in range(I)] for t in range(T)]
    # operand 0: rows of g_y along O; groups = tokens
    op0 = [[sum(int(H[k, m]) * float(gy[t, b * n + m]) for m in range(n))
            for b in range(O // n) for k in range(n)] for t in range(T)]
    # operand 1: columns of w along O; groups = input channels
    op1 = [[sum(int(H[k, m]) * float(w[b * n + m, i]) for m in range(n))
            for b in range(O // n) for k in range(n)] for i in range(I)]
    # operands 2, 3: low-rank rows along T; groups = channels
    op2 = [[sum(int(H[k, m]) * float(gy[b * n + m, c]) for m in range(n))
            for b in range(T // n) for k in keep] for c in range(O)]
    op3 = [[sum(int(H[k, m]) * x[b * n + m][c] for m in range(n))
            for b in range(T // n) for k in keep] for c in range(I)]

    def err_sum(groups, qmax):
        def qerr(v, a):
            if a == 0.0:
                return float(v)
            inv = f32(qmax) / f32(a)
            s = f32(a) / f32(qmax)
            q = 0 if np.isinf(inv) else max(-qmax, min(qmax, round(float(f32(v) * inv))))
            e = f32(v) - f32(s * f32(q))
            return float(e) ** 2
        tensor_a = max(abs(v) for g in groups for v in g)
        tok = sum(qerr(v, max(abs(u) for u in g)) for g in groups for v in g)
        ten = sum(qerr(v, tensor_a) for g in groups for v in g)
        ss = sum(float(v) ** 2 for g in groups for v in g)
        cnt = sum(len(g) for g in groups)
        return [ss, tok, ten, float(cnt)]

    return np.array(err_sum(op0, 7) + err_sum(op1, 7) + err_sum(op2, 127) + err_sum(op3, 127))


@pytest.mark.parametrize("n,r", [(16, 4), (8, 8), (8, 1)])
def test_lqs_stats_match_brute_force(n, r):
    rng = np.random.default_rng(11 + n + r)
    T, O, I = 2 * n, 2 * n, 6
    gy = rng.integers(-40, 41, size=(T, O)).astype(np.float32)
    gy[3] *= 9                                   # one loud token
    w = rng.integers(-30, 31, size=(O, I)).astype(np.float32)
    q = rng.integers(-7, 8, size=(T, I))
    codes = o.pack_int4(q)
    scales = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), size=T)
    got = o.lqs_stats(gy, codes, scales, w, n, r)
    ref = _brute_stats(gy, codes, scales, w, n, r)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=0)


def test_quant_sq_error_within_half_step():
    # |v - s q| <= s / 2 (plus one rounding of s q and of the difference)
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((64, 48)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    for qmax in (7, 127):
        _, s_tok = o.quantize(v, qmax, 1)
        bound_tok = float(np.sum(v.shape[1] * (s_tok.astype(np.float64) / 2) ** 2)) * (1 + 1e-5)
        assert o.quant_sq_error(v, qmax, 1) <= bound_tok
        _, s_ten = o.quantize(v, qmax, None)
        bound_ten = v.size * (float(s_ten[0]) / 2) ** 2 * (1 + 1e-5)
        assert o.quant_sq_error(v, qmax, None) <= bound_ten
        assert o.quant_sq_error(v, qmax, None) > o.quant_sq_error(v, qmax, 1)


def test_equal_absmax_groups_give_equal_errors():
    # every row's absmax is exactly 1: per-token and per-tensor quantizers are
    # the same quantizer, so the errors agree bit for bit
    rng = np.random.default_rng(6)
    v = rng.uniform(-0.99, 0.99, size=(40, 24)).astype(np.float32)
    v[np.arange(40), rng.integers(0, 24, size=40)] = rng.choice([-1.0, 1.0], size=40)
    for qmax in (7, 127):
        assert o.quant_sq_error(v, qmax, 1) == o.quant_sq_error(v, qmax, None)
        assert o.quant_sq_error(v.T, qmax, 0) == o.quant_sq_error(v.T, qmax, None)


def test_zero_operand_has_zero_error():
    z = np.zeros((16, 8), np.float32)
    assert o.quant_sq_error(z, 7, 1) == 0.0 and o.quant_sq_error(z, 127, None) == 0.0


def test_planted_outlier_token_selects_per_token_for_gx():
    rng = np.random.default_rng(7)
    T, O, I, n, r = 64, 32, 16, 16, 4
    gy = rng.standard_normal((T, O)).astype(np.float32)
    gy[10] *= 20.0                               # one token 20x louder
    w = (rng.standard_normal((O, I)) * 0.02).astype(np.float32)
    codes, scales = o.acbp_pack(rng.standard_normal((T, I)).astype(np.float32))
    st = o.lqs_stats(gy, codes, scales, w, n, r)
    (gx_tok, gx_ten), _ = o.lqs_path_errors(st)
    # per tensor, the quiet tokens round to a few codes: several times the error
    assert gx_ten > 4 * gx_tok
    assert o.lqs_select(st)[0] == o.PER_TOKEN
    # a token so loud that its own rounding error dominates both modes' MSE
    # leaves the two within the threshold: an MSE criterion keeps PER_TENSOR
    gy[10] *= 50.0
    st = o.lqs_stats(gy, codes, scales, w, n, r)
    (gx_tok, gx_ten), _ = o.lqs_path_errors(st)
    assert gx_ten < 1.5 * gx_tok and o.lqs_select(st)[0] == o.PER_TENSOR


def test_identical_tokens_select_per_tensor_for_gx():
    # all tokens equal and all w columns equal up to sign: every group of
    # both g_x operands has the same absmax, so the errors tie -> PER_TENSOR
    rng = np.random.default_rng(8)
    T, O, I, n, r = 32, 32, 8, 16, 4
    gy = np.tile(rng.standard_normal((1, O)).astype(np.float32), (T, 1))
    col = rng.standard_normal((O, 1)).astype(np.float32)
    w = (col * rng.choice([-1.0, 1.0], size=(1, I))).astype(np.float32)
    codes, scales = o.acbp_pack(rng.standard_normal((T, I)).astype(np.float32))
    st = o.lqs_stats(gy, codes, scales, w, n, r)
    assert st[1] == st[2] and st[5] == st[6]
    assert o.lqs_select(st)[0] == o.PER_TENSOR


def _stats_with(gx_tok, gx_ten, gw_tok, gw_ten):
    st = np.zeros(16)
    st[[0, 4, 8, 12]] = 1.0
    st[1], st[2] = gx_tok, gx_ten          # operand 1 contributes zero error
    st[9], st[10] = gw_tok, gw_ten
    return st


@pytest.mark.parametrize("ratio,mode", [(1.0, o.PER_TENSOR), (1.49, o.PER_TENSOR),
                                        (1.5, o.PER_TENSOR), (1.51, o.PER_TOKEN),
                                        (40.0, o.PER_TOKEN)])
def test_threshold_rule(ratio, mode):
    st = _stats_with(0.25, 0.25 * ratio, 0.5, 0.5 * ratio)
    assert o.lqs_select(st) == (mode, mode)
    assert o.lqs_select(st, threshold=100.0) == (o.PER_TENSOR, o.PER_TENSOR)


def test_threshold_rule_zero_cases():
    assert o.lqs_select(_stats_with(0.0, 0.0, 0.0, 1e-30)) == (o.PER_TENSOR, o.PER_TOKEN)
    assert o.lqs_select(np.zeros(16)) == (o.PER_TENSOR, o.PER_TENSOR)


def test_stats_counts_and_signs():
    rng = np.random.default_rng(9)
    T, O, I, n, r = 32, 32, 16, 16, 8
    parts = []
    for _ in range(2):
        gy = rng.standard_normal((T, O)).astype(np.float32)
        w = rng.standard_normal((O, I)).astype(np.float32)
        codes, scales = o.acbp_pack(rng.standard_normal((T, I)).astype(np.float32))
        parts.append((gy, codes, scales, w))
    a = o.lqs_stats(*parts[0], n, r)
    b = o.lqs_stats(*parts[1], n, r)
    assert a[3] == T * O and a[7] == O * I and a[11] == T * r // n * O and a[15] == T * r // n * I
    assert np.all(a >= 0) and np.all(b >= 0)
