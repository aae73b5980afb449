"""Plain CPU oracle of the HLQ/HOT linear-layer backward pass.

TEST INFRASTRUCTURE.  This module is the slow, obviously-correct statement of
what the GPU library computes.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the GPU library shares no code
with it and never calls it.

Sources (the pages this follows; cited by title and section):

* [HLQ] "HLQ: Fast and Efficient Backpropagation via Hadamard Low-rank
  Quantization" (Kim, Park; arXiv 2406.15102, sciencestack.ai page).
  TL;DR: the two backward products g_x = g_y . w and g_w = (1/B) gy_bar^T . x_bar,
  4-bit Hadamard quantization (HQ) on g_x, low-rank int8 processing on g_w,
  int4 activation compression (ACBP).  Table of contents, section
  "Hadamard Transform" (body not on the page).  Figure 2 caption ("frequency
  domain with Hadamard transform").
* [HOT-abs] "HOT: Hadamard-based Optimized Training" (Hugging Face paper page),
  abstract: Hadamard quantization and Hadamard low-rank approximation applied
  per backward path, plus activation buffer compression and layer-wise
  quantizer selection.
* [HOT-sum] "HOT: Hadamard-based Optimized Training" (scime.ai summary),
  section "Approach": INT4 Hadamard quantization for gx, Hadamard low-rank
  approximation plus INT8 quantization for gw, stored activations compressed at
  forward time, per-token vs per-tensor quantization chosen per layer.

The pages print no formulas beyond the two TL;DR identities and no worked
example, so every step below states the reading it takes where they are
silent.  The readings (R1..R9) are:

R1  Hadamard matrix: Sylvester order, entries H[i][j] = (-1)^popcount(i & j),
    unnormalised; the single normalising factor 1/n is applied once, in the
    fp64 epilogue.  ([HLQ] section "Hadamard Transform": title only.)
R2  The transform's fp32 operation order is the radix-2 butterfly with
    ascending stage distance h = 1, 2, 4, ..., n/2; pair (k, k+h) with
    (k & h) == 0 becomes (a + b, a - b).  Arithmetic is IEEE fp32 with
    round-to-nearest-even.  (Order is not on the pages; fixing it makes the
    quantized codes unique.)
R3  Blocks are aligned and non-overlapping from index 0; the transformed
    dimension must be a multiple of the block size n.
R4  "Low-rank" keeps, in each block of n tokens, the r rows of H_n with the
    lowest sequency (number of sign changes).  For power-of-two r these are
    the natural-order rows j*(n/r), j = 0..r-1; outputs are stored block by
    block, j ascending.  ([HLQ] TL;DR "low-rank"; Figure 2 "frequency domain".)
R5  Quantizer: symmetric absmax, no zero point.  For a scale group G with
    qmax = 7 (INT4) or 127 (INT8): a = max|v|; a == 0 gives codes 0 and scale
    0; otherwise inv = fl32(qmax / a), s = fl32(a / qmax),
    q = clamp(rne(fl32(v * inv)), -qmax, qmax).  A group so small that
    qmax / a overflows fp32 (a below about qmax / 3.4e38) is treated like a
    zero group for its codes (inv = 0, codes 0) and keeps s = fl32(a / qmax).
    (The pages do not reach this corner; the reading keeps every code finite.)
R6  Scale groups (layer-wise quantizer selection, [HOT-sum] "Approach"):
    PER_TOKEN gives one scale per GEMM output index of each operand (g_x path:
    one per token t of the transformed g_y and one per input channel i of the
    transformed w; g_w path: one per output channel o of the low-rank g_y and
    one per input channel i of the low-rank x).  PER_TENSOR gives one scale
    per operand.  Each path has its own mode.  ACBP is always per token.
R7  The activation x reaches the backward as ACBP codes; it is dequantized as
    fl32(s_x[t] * q[t, i]) before its low-rank transform.
R8  The "1/B" of the g_w identity ([HLQ] TL;DR) is read as two factors: the
    Hadamard normalisation 1/n (always) and an optional mean-reduction 1/T on
    g_w only (argument ``reduction``).
R9  Outputs g_x [T x I] and g_w [O x I] are fp32; the epilogue is evaluated in
    fp64 and rounded once to fp32.
R10 Layer-wise quantizer selection (LQS; [HOT-abs] abstract, [HOT-sum]
    "Approach" and "Limitations": chosen per layer from a calibration set with
    a 50% MSE-difference threshold).  For each of the four GEMM operands (the
    transformed g_y and w of the g_x path, the low-rank g_y and x of the g_w
    path) and each mode, the squared reconstruction error of every element is
    e^2 with e = fl32(v - fl32(s * q)) (codes and scale of reading R5), summed
    in fp64 over the calibration batches together with sum(v^2).  A path's
    error in a mode is the sum over its two operands of SSE / sum(v^2).  The
    path takes PER_TOKEN when its PER_TENSOR error exceeds its PER_TOKEN error
    by more than the threshold (0.5: more than 50% larger), else PER_TENSOR,
    the single-scale quantizer.  (The pages name the threshold, not the error
    measure; this is the plainest reading of "MSE difference".)
"""
from __future__ import annotations

import numpy as np

PER_TOKEN = 0
PER_TENSOR = 1
SUM = 0
MEAN = 1

QMAX_INT4 = 7
QMAX_INT8 = 127


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32; exact (the low 16 bits are 0)."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Hadamard transform ([HLQ] section "Hadamard Transform"; readings R1-R4)
# --------------------------------------------------------------------------

def sylvester_hadamard(n: int) -> np.ndarray:
    """Explicit H_n with H[i][j] = (-1)^popcount(i & j) (reading R1), int64."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.bitwise_and(i, j)
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits = bits >> 1
    return np.where(pop % 2 == 0, 1, -1).astype(np.int64)


def fwht_blocks(v: np.ndarray, n: int, axis: int) -> np.ndarray:
    """Block Walsh-Hadamard transform of ``v`` along ``axis`` (readings R1-R3).

    Every aligned block of ``n`` entries along ``axis`` is replaced by H_n times
    that block, computed with radix-2 butterflies in ascending stage order
    (h = 1, 2, ..., n/2).  The arithmetic is done in ``v``'s own dtype: fp32
    for the quantized path (each add/sub rounds once, RNE), fp64 for the
    quantization-off self-checks.
    """
    if n < 1 or n & (n - 1):
        raise ValueError("block size must be a power of two")
    x = np.moveaxis(np.array(v, copy=True), axis, 0)
    L = x.shape[0]
    if L % n:
        raise ValueError("transformed dimension must be a multiple of the block")
    rest = x.shape[1:]
    x = x.reshape((L // n, n) + rest)          # [block, position, ...]
    h = 1
    while h < n:
        # positions k with (k & h) == 0 pair with k + h
        lo = np.array([k for k in range(n) if k & h == 0])
        a = x[:, lo].copy()
        b = x[:, lo + h].copy()
        x[:, lo] = a + b
        x[:, lo + h] = a - b
        h *= 2
    x = x.reshape((L,) + rest)
    return np.moveaxis(x, 0, axis)


def lowrank_rows(n: int, r: int) -> np.ndarray:
    """Rows of H_n kept by the low-rank step (reading R4): j*(n/r), j < r."""
    if r < 1 or r > n or r & (r - 1):
        raise ValueError("rank must be a power of two in [1, n]")
    return np.arange(r) * (n // r)


def sequency(h: np.ndarray) -> np.ndarray:
    """Number of sign changes along each row of a +-1 matrix."""
    return (h[:, 1:] != h[:, :-1]).sum(axis=1)


def lowrank_transform(v: np.ndarray, n: int, r: int, axis: int = 0) -> np.ndarray:
    """Hadamard low-rank approximation along ``axis`` (HLA; reading R4).

    Full block transform along ``axis`` followed by keeping, in every block,
    the rows j*(n/r) in ascending j.  The result has length L*r/n along
    ``axis``.
    """
    full = fwht_blocks(v, n, axis)
    x = np.moveaxis(full, axis, 0)
    L = x.shape[0]
    keep = (np.arange(L // n)[:, None] * n + lowrank_rows(n, r)[None, :]).reshape(-1)
    return np.moveaxis(x[keep], 0, axis)


# --------------------------------------------------------------------------
# Quantizer (readings R5, R6)
# --------------------------------------------------------------------------

def quantize(v: np.ndarray, qmax: int, reduce_axis):
    """Symmetric absmax quantization of fp32 ``v`` (reading R5).

    ``reduce_axis`` is the axis a scale group runs along (``None``: the whole
    tensor is one group).  Returns (codes int8, scales fp32); scales keep the
    non-reduced axis (or are a 1-element array for the whole tensor).
    """
    v = np.asarray(v, dtype=np.float32)
    if reduce_axis is None:
        a = np.abs(v).max(keepdims=True).reshape(1)
        a_b = a.reshape((1,) * v.ndim)
    else:
        a_b = np.abs(v).max(axis=reduce_axis, keepdims=True)
        a = np.squeeze(a_b, axis=reduce_axis)
    qm = np.float32(qmax)
    zero = a_b == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = np.where(zero, np.float32(0), qm / np.where(zero, np.float32(1), a_b)).astype(np.float32)
        inv = np.where(np.isinf(inv), np.float32(0), inv).astype(np.float32)  # R5 overflow corner
        s = np.where(a == 0, np.float32(0), a / qm).astype(np.float32)
    prod = (v * inv).astype(np.float32)            # one fp32 rounding
    q = np.clip(np.rint(prod), -qmax, qmax)        # rint: round half to even
    return q.astype(np.int8), s.astype(np.float32)


# --------------------------------------------------------------------------
# Activation buffer compression (ACBP): [HLQ] TL;DR, [HOT-abs], [HOT-sum]
# --------------------------------------------------------------------------

def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, element 2k in bits 3:0, 2k+1 in bits 7:4."""
    q = np.asarray(q, dtype=np.int16)
    if q.shape[-1] % 2:
        raise ValueError("last dimension must be even")
    u = (q & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def acbp_pack(x: np.ndarray):
    """Store the layer input as INT4 codes with one fp32 scale per token.

    x [T x I] (fp32 values) -> (codes uint8 [T][I/2], scales fp32 [T]).
    """
    q, s = quantize(np.asarray(x, dtype=np.float32), QMAX_INT4, reduce_axis=1)
    return pack_int4(q), s


def acbp_unpack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantize ACBP codes: x[t, i] = fl32(s[t] * q[t, i]) (reading R7)."""
    q = unpack_int4(codes).astype(np.float32)
    return (np.asarray(scales, dtype=np.float32)[:, None] * q).astype(np.float32)


# --------------------------------------------------------------------------
# Integer GEMM and epilogue ([HLQ] TL;DR "int8-accelerated"; reading R9)
# --------------------------------------------------------------------------

def int_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact integer product a [M x K] . b [K x N] -> int64.

    Evaluated with an fp64 matrix product: every partial sum is an integer of
    magnitude below 2^53, so fp64 represents each one exactly.
    """
    a = np.asarray(a)
    b = np.asarray(b)
    K = a.shape[1]
    bound = K * int(np.abs(a).max(initial=0)) * int(np.abs(b).max(initial=0))
    assert bound < 2 ** 53, "integer GEMM would leave the exact fp64 range"
    return np.rint(a.astype(np.float64) @ b.astype(np.float64)).astype(np.int64)


def _group_axis(mode: int, axis: int):
    if mode == PER_TOKEN:
        return axis
    if mode == PER_TENSOR:
        return None
    raise ValueError("mode must be PER_TOKEN or PER_TENSOR")


def _bcast(s: np.ndarray, axis: int) -> np.ndarray:
    """Scale vector -> broadcastable along the non-reduced axis."""
    s = np.asarray(s, dtype=np.float64)
    if s.size == 1:
        return s.reshape(1, 1)
    return s[:, None] if axis == 0 else s[None, :]


# --------------------------------------------------------------------------
# The backward pass
# --------------------------------------------------------------------------

def _backward_core(gy, x, w, block: int, rank: int, gx_mode: int, gw_mode: int,
                   reduction: int) -> dict:
    """Both paths of the backward for fp32 g_y [T x O], x [T x I] (the
    decoded activation) and w [O x I]; the epilogues are left in fp64
    (gx64, gw64) for the caller to round once.  See linear_backward."""
    T, O = gy.shape
    O2, I = w.shape
    assert O2 == O and x.shape == (T, I)
    n, r = block, rank

    # g_x path: Hadamard along O (the contracted dimension), INT4.
    gy_h = fwht_blocks(gy, n, axis=1)
    w_h = fwht_blocks(w, n, axis=0)
    q_gy, s_gy = quantize(gy_h, QMAX_INT4, _group_axis(gx_mode, 1))
    q_w, s_w = quantize(w_h, QMAX_INT4, _group_axis(gx_mode, 0))
    acc_x = int_matmul(q_gy, q_w)
    gx64 = acc_x.astype(np.float64) * _bcast(s_gy, 0) * _bcast(s_w, 1) / n

    # g_w path: low-rank Hadamard along T (the contracted dimension), INT8.
    gy_l = lowrank_transform(gy, n, r, axis=0)
    x_l = lowrank_transform(x, n, r, axis=0)
    q_gyl, s_gyl = quantize(gy_l, QMAX_INT8, _group_axis(gw_mode, 0))
    q_xl, s_xl = quantize(x_l, QMAX_INT8, _group_axis(gw_mode, 0))
    acc_w = int_matmul(q_gyl.T, q_xl)
    gw64 = acc_w.astype(np.float64) * _bcast(s_gyl, 0) * _bcast(s_xl, 1) / n
    if reduction == MEAN:
        gw64 = gw64 / T
    elif reduction != SUM:
        raise ValueError("reduction must be SUM or MEAN")
    return dict(q_gy=q_gy, s_gy=s_gy, q_w=q_w, s_w=s_w, acc_x=acc_x, gx64=gx64,
                q_gyl=q_gyl, s_gyl=s_gyl, q_xl=q_xl, s_xl=s_xl, acc_w=acc_w, gw64=gw64)


def linear_backward(gy, x_codes, x_scales, w, block: int, rank: int,
                    gx_mode: int = PER_TOKEN, gw_mode: int = PER_TOKEN,
                    reduction: int = SUM) -> dict:
    """HLQ/HOT backward of y = x . w^T for one linear layer.

    gy [T x O] and w [O x I] hold fp32 values (bf16 inputs widened exactly);
    x arrives as ACBP codes [T][I/2] with per-token scales [T].

    g_x path ([HLQ] TL;DR "4-bit HQ for g_x"; [HOT-sum] "Approach"):
      gy_h = H along O of gy (blocks of n), w_h = H along O of w; both
      quantized to INT4; acc_x = q_gy . q_w (int); g_x = acc_x*s_gy*s_w/n.
    g_w path ([HLQ] TL;DR "low-rank, int8-accelerated processing for g_w";
    [HOT-sum] "Approach"):
      gy_l, x_l = low-rank H along T of gy and of dequantized x; both
      quantized to INT8; acc_w = q_gyl^T . q_xl; g_w = acc_w*s*s/n (/T if MEAN).

    Returns every intermediate in its logical layout (codes as int8 values):
      q_gy [T x O], s_gy [T] or [1], q_w [O x I], s_w [I] or [1],
      acc_x [T x I], g_x [T x I],
      q_gyl [T' x O], s_gyl [O] or [1], q_xl [T' x I], s_xl [I] or [1],
      acc_w [O x I], g_w [O x I],  with T' = T*rank/block.
    """
    gy = np.asarray(gy, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    x = acbp_unpack(x_codes, x_scales)
    out = _backward_core(gy, x, w, block, rank, gx_mode, gw_mode, reduction)
    out["g_x"] = out.pop("gx64").astype(np.float32)
    out["g_w"] = out.pop("gw64").astype(np.float32)
    out["x_deq"] = x
    return out


def linear_forward(x, w) -> np.ndarray:
    """y = x . w^T in fp64 (the layer's forward product; ACBP of x is
    :func:`acbp_pack`)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def linear_backward_unquantized(gy, x, w, block: int, rank: int,
                                reduction: int = SUM) -> dict:
    """Quantization-off form of :func:`linear_backward` (self-checks only).

    Same transforms, no ACBP, no quantizer, fp64 throughout.  With
    rank == block this must give back g_x = gy . w and g_w = gy^T . x, since
    H_n^T H_n = n I.
    """
    gy = np.asarray(gy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T = gy.shape[0]
    n = block
    g_x = fwht_blocks(gy, n, axis=1) @ fwht_blocks(w, n, axis=0) / n
    g_w = lowrank_transform(gy, n, rank, axis=0).T @ lowrank_transform(x, n, rank, axis=0) / n
    if reduction == MEAN:
        g_w = g_w / T
    return dict(g_x=g_x, g_w=g_w)


# --------------------------------------------------------------------------
# Ablation variants ([HOT-sum] "Measured effects": the ResNet50 / CIFAR100
# ablation rows, and "Surprising findings": internal and external HLA on the
# activation-gradient path, quantization sensitivity of the weight-gradient
# path)
# --------------------------------------------------------------------------
#
# R12 Each backward path is one GEMM C = A^T-contracted product of two
#     operands over a contracted dimension K (O for g_x, T for g_w).  A
#     variant fixes the operands' transform and quantizer:
#       "hq4"      block Hadamard along K on both operands, INT4 (the method's
#                  g_x path);
#       "q4"       no transform, INT4;
#       "hla8_int" low-rank Hadamard along K on both operands ("internal"
#                  HLA, along the contracted dimension), INT8 (the method's
#                  g_w path);
#       "hla8_ext" low-rank Hadamard along the output dimension of the left
#                  operand (T for g_x, O for g_w: "external" HLA), none on the
#                  right operand, INT8; the GEMM result of r rows per block is
#                  expanded back to n rows by H_low^T / n.
#     The pages' ablation rows list HLA without a quantizer; HOT applies HLA
#     with INT8, so the variants here pair HLA with INT8 and keep integer
#     GEMMs.  A Hadamard along K (hq4, hla8_int) brings the 1/n of R1; q4 none;
#     hla8_ext has its 1/n in the expansion.  Scale groups as R6 (one scale per
#     GEMM output index of each operand, or one per operand).

VARIANTS = ("hq4", "q4", "hla8_int", "hla8_ext")


def expand_lowrank_rows(g, n: int, r: int) -> np.ndarray:
    """(1/n) H_low^T along rows: [B*r x N] -> [B*n x N] in fp64; row k of
    block b is sum_j H[j*n/r][k] * g[b*r + j] / n."""
    h = sylvester_hadamard(n)[lowrank_rows(n, r)].astype(np.float64)   # [r x n]
    g = np.asarray(g, dtype=np.float64)
    B = g.shape[0] // r
    out = np.einsum("jk,bjc->bkc", h, g.reshape(B, r, -1)) / n
    return out.reshape(B * n, -1)


def _variant_operands(a, b, variant: str, n: int, r: int, quant: bool, a_mode: int, b_mode: int):
    """Operands of one path.  a [K x Ma] and b [K x Nb] with K (the
    contracted dimension) along axis 0.  Returns (qa, sa, qb, sb, alpha):
    quantized codes (or the fp64 values when quant is False) along with their
    scales (1 when unquantized), and the factor of the product."""
    def tr(v, kind):
        if kind == "h":
            return fwht_blocks(v, n, 0)
        if kind == "low_k":
            return lowrank_transform(v, n, r, 0)
        if kind == "low_m":
            return lowrank_transform(v, n, r, 1)
        return v
    kinds = {"hq4": ("h", "h", QMAX_INT4, 1.0 / n), "q4": ("none", "none", QMAX_INT4, 1.0),
             "hla8_int": ("low_k", "low_k", QMAX_INT8, 1.0 / n),
             "hla8_ext": ("low_m", "none", QMAX_INT8, 1.0)}
    if variant not in kinds:
        raise ValueError(f"unknown variant {variant!r}")
    ka, kb, qmax, alpha = kinds[variant]
    va, vb = tr(a, ka), tr(b, kb)
    if not quant:
        return va, np.ones(1), vb, np.ones(1), alpha
    qa, sa = quantize(va, qmax, _group_axis(a_mode, 0))
    qb, sb = quantize(vb, qmax, _group_axis(b_mode, 0))
    return qa, sa, qb, sb, alpha


def linear_backward_variant(gy, x_codes, x_scales, w, block: int, rank: int, gx_variant: str,
                            gw_variant: str, gx_mode: int = PER_TOKEN, gw_mode: int = PER_TOKEN,
                            reduction: int = SUM, quant: bool = True) -> dict:
    """The backward with one variant per path (reading R12).  Inputs as
    :func:`linear_backward`; ``quant=False`` skips the quantizers (fp64
    throughout, self-checks).  Returns the codes / scales of each operand
    (qa_x, sa_x, qb_x, sb_x; qa_w, sa_w, qb_w, sb_w, each K-contracted along
    axis 0), the INT32 sums acc_x [T' or T x I] and acc_w [O' or O x I], and
    g_x [T x I], g_w [O x I] (fp64 epilogue and expansion, rounded once)."""
    dt = np.float32 if quant else np.float64
    gy = np.asarray(gy, dtype=dt)
    w = np.asarray(w, dtype=dt)
    x = acbp_unpack(x_codes, x_scales).astype(dt)
    n, r = block, rank
    T = gy.shape[0]
    out = {}
    # g_x = gy . w: K = O; a = gy^T [O x T], b = w [O x I]
    qa, sa, qb, sb, alpha = _variant_operands(gy.T, w, gx_variant, n, r, quant, gx_mode, gx_mode)
    acc = int_matmul(qa.T, qb) if quant else qa.T @ qb
    g = acc.astype(np.float64) * _bcast(sa, 0) * _bcast(sb, 1) * alpha
    if gx_variant == "hla8_ext":
        g = expand_lowrank_rows(g, n, r)
    out.update(qa_x=qa, sa_x=sa, qb_x=qb, sb_x=sb, acc_x=acc, g_x=g.astype(dt))
    # g_w = gy^T . x: K = T; a = gy [T x O], b = x [T x I]
    qa, sa, qb, sb, alpha = _variant_operands(gy, x, gw_variant, n, r, quant, gw_mode, gw_mode)
    acc = int_matmul(qa.T, qb) if quant else qa.T @ qb
    g = acc.astype(np.float64) * _bcast(sa, 0) * _bcast(sb, 1) * alpha
    if gw_variant == "hla8_ext":
        g = expand_lowrank_rows(g, n, r)
    if reduction == MEAN:
        g = g / T
    elif reduction != SUM:
        raise ValueError("reduction must be SUM or MEAN")
    out.update(qa_w=qa, sa_w=sa, qb_w=qb, sb_w=sb, acc_w=acc, g_w=g.astype(dt))
    return out


# --------------------------------------------------------------------------
# Convolution layers ([HLQ] abstract: backpropagation of convolutional and
# linear layers; [HOT-sum] "Key results": ResNet-50 at batch size 256)
# --------------------------------------------------------------------------
#
# R11 A convolution y[n,p,q,o] = sum_{r,s,c} x[n, p*st - pad + r, q*st - pad + s, c]
#     * w[o,r,s,c] (NHWC activations, OHWI weights, zero padding) is the
#     linear layer y = im2col(x) . w^T with tokens t = (n, p, q) and input
#     features i = (r, s, c) (column (r*S + s)*C + c).  Its HLQ/HOT backward is
#     the linear backward on (g_y, im2col(x), w): ACBP stores the convolution
#     input x itself (per pixel (n, h, w), over its C channels) and im2col
#     gathers the decoded values; g_w [O][R][S][C] is the linear g_w; g_x is
#     col2im of the linear g_x, the sum over the taps (r, s) that read each
#     input pixel, rounded once to fp32 (as R9).  With per-tensor g_x scales
#     every term shares the scale pair, and the sum is taken exactly as the
#     integer col2im of the accumulators times the scales / n; with
#     per-token scales the terms are summed in fp64.


def conv_out_size(H: int, R: int, stride: int, pad: int) -> int:
    """Output rows of a convolution along one spatial axis."""
    return (H + 2 * pad - R) // stride + 1


def im2col(x, R: int, S: int, stride: int, pad: int) -> np.ndarray:
    """x [N, H, W, C] -> [N*P*Q, R*S*C]: row (n, p, q), column (r*S + s)*C + c
    holds x[n, p*stride - pad + r, q*stride - pad + s, c], 0 outside the image."""
    x = np.asarray(x)
    N, H, W, C = x.shape
    P, Q = conv_out_size(H, R, stride, pad), conv_out_size(W, S, stride, pad)
    cols = np.zeros((N, P, Q, R, S, C), dtype=x.dtype)
    for r in range(R):
        for s in range(S):
            for p in range(P):
                h = p * stride - pad + r
                if not 0 <= h < H:
                    continue
                for q in range(Q):
                    w_ = q * stride - pad + s
                    if 0 <= w_ < W:
                        cols[:, p, q, r, s, :] = x[:, h, w_, :]
    return cols.reshape(N * P * Q, R * S * C)


def col2im(cols, N: int, H: int, W: int, C: int, R: int, S: int, stride: int,
           pad: int) -> np.ndarray:
    """Adjoint of im2col: [N*P*Q, R*S*C] -> [N, H, W, C], each input pixel the
    sum of the entries im2col copied it to (in the dtype of ``cols``: fp64 for
    gradients, int64 for integer accumulators)."""
    P, Q = conv_out_size(H, R, stride, pad), conv_out_size(W, S, stride, pad)
    c6 = np.asarray(cols).reshape(N, P, Q, R, S, C)
    g = np.zeros((N, H, W, C), dtype=c6.dtype)
    for r in range(R):
        for s in range(S):
            for p in range(P):
                h = p * stride - pad + r
                if not 0 <= h < H:
                    continue
                for q in range(Q):
                    w_ = q * stride - pad + s
                    if 0 <= w_ < W:
                        g[:, h, w_, :] += c6[:, p, q, r, s, :]
    return g


def conv_backward(gy, x_codes, x_scales, w, N: int, H: int, W: int, C: int, R: int, S: int,
                  stride: int, pad: int, block: int, rank: int, gx_mode: int = PER_TOKEN,
                  gw_mode: int = PER_TOKEN, reduction: int = SUM) -> dict:
    """HLQ/HOT backward of one convolution (reading R11).

    gy [N*P*Q x O] (rows (n, p, q)), x_codes [N*H*W][C/2] and x_scales [N*H*W]
    (ACBP of the input, per pixel), w [O x R*S*C] (OHWI).  Returns the linear
    backward's intermediates on (gy, im2col(x), w) (q_gy, s_gy, q_w, s_w,
    q_gyl, s_gyl, q_xl, s_xl, acc_w, g_w, with acc_x_col the linear g_x
    accumulators) and g_x [N*H*W x C] = col2im of the fp64 linear g_x, rounded
    once; acc_x [N*H*W x C] = col2im of acc_x_col (int64), the integer sums a
    per-tensor g_x epilogue scales.
    """
    gy = np.asarray(gy, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    xd = acbp_unpack(x_codes, x_scales).reshape(N, H, W, C)
    cols = im2col(xd, R, S, stride, pad)
    out = _backward_core(gy, cols, w, block, rank, gx_mode, gw_mode, reduction)
    out["acc_x_col"] = out.pop("acc_x")
    out["acc_x"] = col2im(out["acc_x_col"], N, H, W, C, R, S, stride, pad).reshape(N * H * W, C)
    gx64 = out.pop("gx64")
    if gx_mode == PER_TENSOR:
        # one scale pair for every term: the exact sum over the taps is the
        # integer sum times the scales (so exact cancellations give exact 0)
        gx = out["acc_x"].astype(np.float64) * _bcast(out["s_gy"], 0) * _bcast(out["s_w"], 1) / block
    else:
        gx = col2im(gx64, N, H, W, C, R, S, stride, pad).reshape(N * H * W, C)
    out["g_x"] = gx.astype(np.float32)
    out["g_w"] = out.pop("gw64").astype(np.float32)
    out["x_col"] = cols
    return out


def conv_backward_unquantized(gy, x, w, N: int, H: int, W: int, C: int, R: int, S: int,
                              stride: int, pad: int, block: int, rank: int,
                              reduction: int = SUM) -> dict:
    """Quantization-off form of :func:`conv_backward` (self-checks): fp64
    transforms and products, x given directly as [N, H, W, C]."""
    cols = im2col(np.asarray(x, dtype=np.float64), R, S, stride, pad)
    lin = linear_backward_unquantized(gy, cols, w, block, rank, reduction)
    gx = col2im(lin["g_x"], N, H, W, C, R, S, stride, pad)
    return dict(g_x=gx.reshape(N * H * W, C), g_w=lin["g_w"])


# --------------------------------------------------------------------------
# Layer-wise quantizer selection ([HOT-abs] abstract; [HOT-sum] "Approach",
# "Limitations"; reading R10)
# --------------------------------------------------------------------------

LQS_THRESHOLD = 0.5
LQS_OPERANDS = ("H.g_y", "H.w", "lowrank g_y", "lowrank x")


def lqs_operands(gy, x_codes, x_scales, w, block: int, rank: int):
    """The four transformed GEMM operands as (values fp32, qmax, group axis).

    The group axis is the axis one PER_TOKEN scale runs along (reading R6):
    along O for each token of H.g_y, along O for each input channel of H.w,
    along T' for each channel of the low-rank g_y and x.
    """
    gy = np.asarray(gy, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    n, r = block, rank
    x = acbp_unpack(x_codes, x_scales)
    return [(fwht_blocks(gy, n, axis=1), QMAX_INT4, 1),
            (fwht_blocks(w, n, axis=0), QMAX_INT4, 0),
            (lowrank_transform(gy, n, r, axis=0), QMAX_INT8, 0),
            (lowrank_transform(x, n, r, axis=0), QMAX_INT8, 0)]


def quant_sq_error(v: np.ndarray, qmax: int, reduce_axis) -> float:
    """Sum over v of e^2 (fp64), e = fl32(v - fl32(s * q)) with the codes and
    scales of :func:`quantize` for that grouping (reading R10)."""
    v = np.asarray(v, dtype=np.float32)
    q, s = quantize(v, qmax, reduce_axis)
    if reduce_axis is None:
        sb = s.reshape((1,) * v.ndim)
    else:
        sb = np.expand_dims(s, reduce_axis)
    deq = (sb * q.astype(np.float32)).astype(np.float32)
    e = (v - deq).astype(np.float32)
    return float(np.sum(e.astype(np.float64) ** 2))


def lqs_stats(gy, x_codes, x_scales, w, block: int, rank: int) -> np.ndarray:
    """LQS statistics of one calibration batch: 16 fp64 values, four per
    operand k (order of LQS_OPERANDS): [4k] sum(v^2), [4k+1] SSE PER_TOKEN,
    [4k+2] SSE PER_TENSOR, [4k+3] element count.  Batches add up."""
    out = np.zeros(16, dtype=np.float64)
    for k, (v, qmax, axis) in enumerate(lqs_operands(gy, x_codes, x_scales, w, block, rank)):
        out[4 * k] = float(np.sum(v.astype(np.float64) ** 2))
        out[4 * k + 1] = quant_sq_error(v, qmax, axis)
        out[4 * k + 2] = quant_sq_error(v, qmax, None)
        out[4 * k + 3] = float(v.size)
    return out


def lqs_path_errors(stats) -> tuple:
    """((E_tok, E_ten) of the g_x path, (E_tok, E_ten) of the g_w path):
    per mode, the sum over the path's two operands of SSE / sum(v^2), each
    term 0 for an all-zero operand."""
    st = np.asarray(stats, dtype=np.float64)

    def rel(k, col):
        ss = st[4 * k]
        return 0.0 if ss == 0.0 else float(st[4 * k + col] / ss)

    gx = (rel(0, 1) + rel(1, 1), rel(0, 2) + rel(1, 2))
    gw = (rel(2, 1) + rel(3, 1), rel(2, 2) + rel(3, 2))
    return gx, gw


def lqs_select(stats, threshold: float = LQS_THRESHOLD) -> tuple:
    """(gx_mode, gw_mode): PER_TOKEN for a path whose PER_TENSOR error is more
    than (1 + threshold) times its PER_TOKEN error, else PER_TENSOR."""
    modes = []
    for e_tok, e_ten in lqs_path_errors(stats):
        modes.append(PER_TOKEN if e_ten > (1.0 + threshold) * e_tok else PER_TENSOR)
    return tuple(modes)


def rel_fro(a, b) -> float:
    """||a - b||_F / ||b||_F in fp64 (0 when both are zero)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    num = np.linalg.norm(a - b)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


def max_rel_err(a, b, tiny: float) -> float:
    """max_i |a_i - b_i| / max(|b_i|, tiny) in fp64: the element-wise relative
    error, measured absolutely (in units of ``tiny``) where the reference is
    below ``tiny``.  0 for empty arrays."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError("shapes differ")
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), float(tiny))))


__all__ = [
    "PER_TOKEN", "PER_TENSOR", "SUM", "MEAN", "QMAX_INT4", "QMAX_INT8",
    "bf16_bits_to_f32",
    "sylvester_hadamard", "fwht_blocks", "lowrank_rows", "sequency",
    "lowrank_transform", "quantize", "pack_int4", "unpack_int4", "acbp_pack",
    "acbp_unpack", "int_matmul", "linear_backward", "linear_forward",
    "linear_backward_unquantized", "rel_fro", "max_rel_err", "conv_out_size", "im2col",
    "col2im", "conv_backward", "conv_backward_unquantized", "VARIANTS",
    "expand_lowrank_rows", "linear_backward_variant", "LQS_THRESHOLD", "LQS_OPERANDS",
    "lqs_operands", "quant_sq_error", "lqs_stats", "lqs_path_errors", "lqs_select",
]
