"""Pins of the oracle's ablation variants (reading R12) against facts that do
not come from them: the method's own path (bit for bit), closed forms with
the quantizer off (full Hadamard: exact products; low rank along a dimension:
the group-average projector on that dimension), a brute-force quantizer and a
hand-worked expansion.  Source: "HOT: Hadamard-based Optimized Training"
(scime.ai summary, "Measured effects" ablation rows, "Surprising findings")."""
import json
import os

import numpy as np
import pytest

import oracle as o

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def _inputs(seed=0, T=64, I=24, O=48):
    rng = np.random.default_rng(seed)
    gy = rng.standard_normal((T, O)).astype(np.float32)
    x = rng.standard_normal((T, I)).astype(np.float32)
    w = (0.05 * rng.standard_normal((O, I))).astype(np.float32)
    c, s = o.acbp_pack(x)
    return gy, c, s, w


@pytest.mark.parametrize("modes", [(0, 0), (0, 1), (1, 1)])
def test_method_variants_equal_the_method(modes):
    # hq4 on g_x and internal HLA with INT8 on g_w are the method itself
    gy, c, s, w = _inputs(1)
    ref = o.linear_backward(gy, c, s, w, 16, 4, *modes)
    v = o.linear_backward_variant(gy, c, s, w, 16, 4, "hq4", "hla8_int", *modes)
    for a, b in (("acc_x", "acc_x"), ("acc_w", "acc_w"), ("g_x", "g_x"), ("g_w", "g_w")):
        assert np.array_equal(v[a], ref[b]), a


def _projector(L, n, r):
    """Group average over consecutive groups of n/r along a length-L axis."""
    g = n // r
    P = np.zeros((L, L))
    for a in range(0, L, g):
        P[a:a + g, a:a + g] = 1.0 / g
    return P


def test_quant_off_closed_forms():
    n, r, T, I, O = 16, 4, 64, 12, 32
    rng = np.random.default_rng(2)
    gy = rng.standard_normal((T, O))
    xq = rng.integers(-7, 8, (T, I))
    codes, sc = o.pack_int4(xq), np.ones(T, np.float32)
    x = xq.astype(np.float64)
    w = rng.standard_normal((O, I))
    gx_exact, gw_exact = gy @ w, gy.T @ x
    PT, PO = _projector(T, n, r), _projector(O, n, r)

    def run(vx, vw):
        return o.linear_backward_variant(gy, codes, sc, w, n, r, vx, vw, quant=False)

    for v in ("hq4", "q4"):          # a full Hadamard or none: exact products
        out = run(v, v)
        np.testing.assert_allclose(out["g_x"], gx_exact, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out["g_w"], gw_exact, rtol=1e-12, atol=1e-12)
    out = run("hla8_int", "hla8_int")   # low rank along the contracted dimension
    np.testing.assert_allclose(out["g_x"], gy @ PO @ w, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["g_w"], gy.T @ PT @ x, rtol=1e-12, atol=1e-12)
    out = run("hla8_ext", "hla8_ext")   # low rank along an output dimension
    np.testing.assert_allclose(out["g_x"], PT @ gx_exact, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["g_w"], PO @ gw_exact, rtol=1e-12, atol=1e-12)


def _brute_quant_tok(v, qmax):
    """Per-column (output index) symmetric absmax quantizer by brute force on
    a K x M operand."""
    q = np.zeros(v.shape, np.int64)
    s = np.zeros(v.shape[1], np.float32)
    for m in range(v.shape[1]):
        a = max(abs(float(t)) for t in v[:, m])
        if a == 0:
            continue
        inv = np.float32(np.float32(qmax) / np.float32(a))
        s[m] = np.float32(np.float32(a) / np.float32(qmax))
        for k in range(v.shape[0]):
            p = float(np.float32(v[k, m] * inv))
            q[k, m] = int(max(-qmax, min(qmax, round(p))))   # round(): half to even
    return q, s


def test_q4_codes_by_brute_force():
    gy, c, s, w = _inputs(3, T=32, I=8, O=16)
    out = o.linear_backward_variant(gy, c, s, w, 16, 4, "q4", "q4")
    q, sc = _brute_quant_tok(gy.T, 7)
    assert np.array_equal(out["qa_x"], q) and np.array_equal(out["sa_x"], sc)
    q, sc = _brute_quant_tok(o.acbp_unpack(c, s), 7)
    assert np.array_equal(out["qb_w"], q) and np.array_equal(out["sb_w"], sc)


def test_expand_lowrank_golden():
    g = GOLDEN["expand_lowrank_n4_r2"]
    out = o.expand_lowrank_rows(np.array(g["G"], np.float64), g["n"], g["r"])
    assert out.tolist() == g["out"]


def test_mean_reduction_scales_every_gw_variant():
    gy, c, s, w = _inputs(4)
    for v in o.VARIANTS:
        a = o.linear_backward_variant(gy, c, s, w, 16, 4, "q4", v, reduction=o.SUM)
        b = o.linear_backward_variant(gy, c, s, w, 16, 4, "q4", v, reduction=o.MEAN)
        np.testing.assert_allclose(b["g_w"], a["g_w"] / gy.shape[0], rtol=3e-7)
