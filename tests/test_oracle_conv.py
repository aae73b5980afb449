"""Pins of the oracle's convolution form (im2col / col2im around the linear
backward) against facts that do not come from it: element-by-element
definitions, the adjoint identity, direct convolution gradients and a
hand-worked example.  Sources: "HLQ: Fast and Efficient Backpropagation via
Hadamard Low-rank Quantization" (abstract: convolutional and linear layers);
"HOT: Hadamard-based Optimized Training" (scime.ai summary, "Key results":
ResNet-50 at batch 256)."""
import json
import os

import numpy as np
import pytest

import oracle as o

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))
GEOMS = [  # N, H, W, C, R, S, stride, pad
    (2, 5, 4, 3, 3, 3, 1, 1), (1, 7, 6, 2, 3, 2, 2, 1), (2, 4, 4, 1, 1, 1, 1, 0),
    (1, 6, 5, 2, 2, 3, 2, 0), (1, 5, 5, 2, 5, 5, 1, 2)]


def _brute_im2col(x, R, S, st, pad):
    N, H, W, C = x.shape
    P, Q = o.conv_out_size(H, R, st, pad), o.conv_out_size(W, S, st, pad)
    out = np.zeros((N * P * Q, R * S * C))
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                for r in range(R):
                    for s in range(S):
                        for c in range(C):
                            h, w = p * st - pad + r, q * st - pad + s
                            if 0 <= h < H and 0 <= w < W:
                                out[(n * P + p) * Q + q, (r * S + s) * C + c] = x[n, h, w, c]
    return out


@pytest.mark.parametrize("geom", GEOMS)
def test_im2col_matches_definition(geom):
    N, H, W, C, R, S, st, pad = geom
    x = np.random.default_rng(1).integers(-9, 10, (N, H, W, C)).astype(np.float64)
    assert np.array_equal(o.im2col(x, R, S, st, pad), _brute_im2col(x, R, S, st, pad))


@pytest.mark.parametrize("geom", GEOMS)
def test_col2im_is_the_adjoint_of_im2col(geom):
    # <im2col(x), Y> = <x, col2im(Y)>, exact on integers; catches a wrong
    # offset, a dropped tap or a misplaced padding in either direction
    N, H, W, C, R, S, st, pad = geom
    rng = np.random.default_rng(2)
    x = rng.integers(-9, 10, (N, H, W, C)).astype(np.float64)
    P, Q = o.conv_out_size(H, R, st, pad), o.conv_out_size(W, S, st, pad)
    Y = rng.integers(-9, 10, (N * P * Q, R * S * C)).astype(np.float64)
    lhs = float(np.sum(o.im2col(x, R, S, st, pad) * Y))
    rhs = float(np.sum(x * o.col2im(Y, N, H, W, C, R, S, st, pad)))
    assert lhs == rhs


def _direct_conv_grads(gy, x, w, st, pad):
    """Gradients of y[n,p,q,o] = sum x[n, p*st-pad+r, q*st-pad+s, c] w[o,r,s,c]
    by direct loops (no im2col)."""
    N, H, W, C = x.shape
    O, R, S, _ = w.shape
    P, Q = gy.shape[1], gy.shape[2]
    gx = np.zeros_like(x)
    gw = np.zeros_like(w)
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                for r in range(R):
                    for s in range(S):
                        h, ww = p * st - pad + r, q * st - pad + s
                        if 0 <= h < H and 0 <= ww < W:
                            gx[n, h, ww, :] += gy[n, p, q, :] @ w[:, r, s, :]
                            gw[:, r, s, :] += np.outer(gy[n, p, q, :], x[n, h, ww, :])
    return gx, gw


@pytest.mark.parametrize("geom", [(2, 6, 6, 4, 3, 3, 1, 1), (1, 8, 8, 2, 3, 3, 2, 1),
                                  (2, 5, 5, 3, 1, 1, 1, 0)])
def test_conv_exact_recovery_quant_off_full_rank(geom):
    # quantizer off and rank = block: H^T H = n I, so the backward must give
    # the convolution's exact gradients (integers: bit-equal)
    N, H, W, C, R, S, st, pad = geom
    O = 16
    P, Q = o.conv_out_size(H, R, st, pad), o.conv_out_size(W, S, st, pad)
    n = next(b for b in (16, 8, 4, 2, 1) if (N * P * Q) % b == 0)
    rng = np.random.default_rng(3)
    gy = rng.integers(-5, 6, (N, P, Q, O)).astype(np.float64)
    x = rng.integers(-5, 6, (N, H, W, C)).astype(np.float64)
    w = rng.integers(-5, 6, (O, R, S, C)).astype(np.float64)
    out = o.conv_backward_unquantized(gy.reshape(-1, O), x, w.reshape(O, -1), N, H, W, C, R, S,
                                      st, pad, n, n)
    gx, gw = _direct_conv_grads(gy, x, w, st, pad)
    assert np.array_equal(out["g_x"], gx.reshape(-1, C))
    assert np.array_equal(out["g_w"], gw.reshape(O, -1))


def test_conv_golden():
    g = GOLDEN["conv_2x2_on_3x3"]
    x = np.array(g["x"], np.float64).reshape(1, 3, 3, 1)
    gy = np.array(g["gy"], np.float64).reshape(4, 1)
    w = np.array(g["w"], np.float64).reshape(1, 4)
    # block 1 (H_1 = [1]): O = 1 admits no larger block; the geometry is under test
    out = o.conv_backward_unquantized(gy, x, w, 1, 3, 3, 1, 2, 2, 1, 0, 1, 1)
    assert out["g_w"].reshape(2, 2).tolist() == g["g_w"]
    assert out["g_x"].reshape(3, 3).tolist() == g["g_x"]


def test_conv_backward_is_linear_backward_on_im2col():
    # the quantized conv backward: every code, scale and g_w of the linear
    # backward on the gathered decoded input, and g_x its col2im (integer
    # accumulators summed exactly, fp64 gradient rounded once)
    N, H, W, C, R, S, st, pad, O, n, r = 2, 8, 8, 8, 3, 3, 1, 1, 32, 16, 4
    rng = np.random.default_rng(4)
    P, Q = o.conv_out_size(H, R, st, pad), o.conv_out_size(W, S, st, pad)
    gy = rng.standard_normal((N * P * Q, O)).astype(np.float32)
    x = np.maximum(rng.standard_normal((N * H * W, C)), 0).astype(np.float32)
    w = (0.1 * rng.standard_normal((O, R * S * C))).astype(np.float32)
    codes, sc = o.acbp_pack(x)
    out = o.conv_backward(gy, codes, sc, w, N, H, W, C, R, S, st, pad, n, r,
                          o.PER_TENSOR, o.PER_TOKEN)
    cols = o.im2col(o.acbp_unpack(codes, sc).reshape(N, H, W, C), R, S, st, pad)
    from oracle import hlq_oracle as ho
    lin = ho._backward_core(gy, cols, w, n, r, o.PER_TENSOR, o.PER_TOKEN, o.SUM)
    for k in ("q_gy", "s_gy", "q_w", "s_w", "q_gyl", "s_gyl", "q_xl", "s_xl", "acc_w"):
        assert np.array_equal(out[k], lin[k]), k
    assert np.array_equal(out["g_w"], lin["gw64"].astype(np.float32))
    acc = o.col2im(lin["acc_x"], N, H, W, C, R, S, st, pad).reshape(-1, C)
    assert np.array_equal(out["acc_x"], acc)
    # per-tensor g_x: col2im of the accumulators times the two scales / n
    ref = (acc.astype(np.float64) * float(out["s_gy"][0]) * float(out["s_w"][0]) / n)
    assert np.array_equal(out["g_x"], ref.astype(np.float32))
