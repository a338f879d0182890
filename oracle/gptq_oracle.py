"""Plain CPU oracle for one-shot GPTQ quantization of a single linear layer.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
definition that the HIP library is checked against.  It shares no code with
the HIP path, and nothing on the product path imports it.

Everything here follows the pages' statement of the method:

* GPTQ knowledge note, "How It Works": for each linear layer the recorded
  inputs X give the Hessian H = 2XX^T of the layer-output reconstruction
  loss; after a column is quantized, inverse-Hessian information decides how
  the still-unquantized columns are adjusted; all rows follow one column
  order; 128-column blocks accumulate corrections before a global update; a
  damped Cholesky formulation supplies the correction rows.
* Wiki "GPTQ", "Technical Approach": low-bit grid (4/3/2 bits) with
  group-wise quantization, each group having its own scaling factor.
* Daily Papers page, GPTQ abstract: 2-bit and ternary grids.
* Daily Papers page, abstract on GPTQ and Babai's nearest plane algorithm:
  the rounding errors are propagated to the not-yet-processed entries
  through a triangular feedback matrix (used by the tests as a pin).

Precision: H, the damped inverse factor U and the error propagation are
float64.  The few operations that decide a code (grid range, scale, zero
point, the division w/s and the rounding) are specified in IEEE float32 with
round-half-to-even, and are evaluated here with numpy float32 arithmetic, so
that the GPU kernels can reproduce them bit for bit.  Where the pages are
silent the reading taken is stated next to the code that implements it.

Layouts: W is out x in (rows x columns, columns are the input features that
are swept); X is tokens x in.  "Processing order" is the column order after
the optional act-order permutation.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
(closed forms, hand-worked fixtures under tests/golden/, brute force,
Babai's nearest plane algorithm, a conditional least-squares definition that
does not use U, and an exact loss identity).
"""
from __future__ import annotations

import numpy as np
import scipy.linalg
import scipy.linalg.lapack

F32 = np.float32
F64 = np.float64


class NotPositiveDefinite(ValueError):
    """The damped Hessian is not positive definite.

    ``index`` is the 1-based position (in the factored matrix) of the first
    non-positive pivot, LAPACK style.
    """

    def __init__(self, index: int):
        super().__init__(f"damped Hessian not positive definite (pivot {index})")
        self.index = index


# ---------------------------------------------------------------------------
# a1: Hessian.  GPTQ knowledge note, "How It Works": H = 2 X X^T over the
# recorded layer inputs.  With X stored tokens x n this is H = 2 X^T X.
# ---------------------------------------------------------------------------
def hessian(X, alpha: float = 2.0) -> np.ndarray:
    """H = alpha * X^T X in float64 (X is tokens x n, already dtype-rounded)."""
    X64 = np.asarray(X, dtype=F64)
    return alpha * (X64.T @ X64)


def hessian_rows(X, rows, alpha: float = 2.0, chunk: int = 16384) -> np.ndarray:
    """Rows ``rows`` of H = alpha * X^T X, float64, streaming over tokens."""
    X = np.asarray(X)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, X.shape[1]), dtype=F64)
    for t0 in range(0, X.shape[0], chunk):
        Xc = np.asarray(X[t0:t0 + chunk], dtype=F64)
        out += Xc[:, rows].T @ Xc
    return alpha * out


# ---------------------------------------------------------------------------
# a2: act-order permutation and damping.
# The pages give neither: columns are ordered by descending diag(H) (the
# act-order option of the workload definitions) with ties kept in ascending
# original index (a stable sort), and the damping constant is a parameter
# lambda = damp_rel * mean(diag H) added after permutation (GPTQ knowledge
# note, "How It Works", only says the Cholesky formulation is damped).
# ---------------------------------------------------------------------------
def act_order_perm(H) -> np.ndarray:
    """Stable argsort of diag(H), descending; ties keep ascending index."""
    d = np.diag(np.asarray(H, dtype=F64))
    n = d.size
    # Explicit ordering key: (-d, index).  lexsort sorts by the last key first.
    return np.lexsort((np.arange(n), -d)).astype(np.int64)


def damp_and_permute(H, perm, damp_rel: float):
    """Return (H_d, lam) with H_d = H[perm][:, perm] + lam * I."""
    H = np.asarray(H, dtype=F64)
    n = H.shape[0]
    perm = np.arange(n) if perm is None else np.asarray(perm, dtype=np.int64)
    lam = float(damp_rel) * float(np.mean(np.diag(H)))
    Hd = H[np.ix_(perm, perm)].copy()
    Hd[np.diag_indices(n)] += lam
    return Hd, lam


# ---------------------------------------------------------------------------
# a3: the damped inverse-Hessian factor.  U is upper triangular with positive
# diagonal and U^T U = H_d^{-1}; row j of U divided by U_jj is the correction
# row used when column j is quantized (GPTQ knowledge note, "How It Works":
# "a damped Cholesky formulation supplies stable correction rows").
# Plain definition: invert H_d (via its Cholesky factor), then take the upper
# Cholesky factor of the inverse.
# ---------------------------------------------------------------------------
def _potrf(A, lower: bool) -> np.ndarray:
    """LAPACK Cholesky of the symmetric A read from one triangle; the other
    triangle of the result is zero.  A failure at leading minor k raises
    NotPositiveDefinite(k) (1-based)."""
    c, info = scipy.linalg.lapack.dpotrf(A, lower=1 if lower else 0, clean=1)
    if info > 0:
        raise NotPositiveDefinite(int(info))
    if info < 0:
        raise ValueError(f"dpotrf argument {-info}")
    return c


def inverse_cholesky_upper(Hd) -> np.ndarray:
    """U upper, U^T U = Hd^{-1}.  Raises NotPositiveDefinite."""
    Hd = np.asarray(Hd, dtype=F64)
    n = Hd.shape[0]
    if n == 0:
        return np.zeros((0, 0), dtype=F64)
    if not np.all(np.isfinite(Hd)):
        raise NotPositiveDefinite(1)
    L = _potrf(Hd, lower=True)                       # H_d = L L^T
    inv, info = scipy.linalg.lapack.dpotri(L, lower=1)  # lower triangle of H_d^{-1}
    if info != 0:
        raise NotPositiveDefinite(max(1, int(info)))
    # The upper triangle of inv^T is the lower triangle of H_d^{-1}.
    return np.ascontiguousarray(_potrf(inv.T, lower=False))  # H_d^{-1} = U^T U


# ---------------------------------------------------------------------------
# a4: grid parameters.  Wiki "GPTQ", "Technical Approach": group-wise
# quantization, each group with its own scaling factor, on a uniform low-bit
# grid (GPTQ knowledge note, "Common Confusions": a fixed low-bit grid shared
# with round-to-nearest).  Readings taken (the pages are silent):
#   * asymmetric min-max grid with an integer zero point;
#   * the range always contains 0: xmin = min(0, min w), xmax = max(0, max w);
#   * an all-zero group uses the range [-1, 1];
#   * float32 arithmetic, IEEE division, round half to even:
#       s = fl32(fl32(xmax - xmin) / maxq),  z = clamp(rint(fl32(-xmin / s)), 0, maxq).
# ---------------------------------------------------------------------------
def grid_params(vals, maxq: int):
    """Per-row (scale, zero) of the rows of ``vals`` (rows x group), float32."""
    v = np.asarray(vals, dtype=F32)
    if v.ndim == 1:
        v = v[None, :]
    xmin = np.minimum(v.min(axis=1), F32(0))
    xmax = np.maximum(v.max(axis=1), F32(0))
    degenerate = xmax == xmin
    xmin = np.where(degenerate, F32(-1), xmin).astype(F32)
    xmax = np.where(degenerate, F32(1), xmax).astype(F32)
    s = ((xmax - xmin) / F32(maxq)).astype(F32)
    z = np.rint((-xmin) / s).astype(F32)
    z = np.clip(z, F32(0), F32(maxq)).astype(F32)
    return s, z


def quantize_values(w, s, z, maxq: int, clip: bool = True):
    """Codes c = clamp(rint(fl32(w / s)) + z, 0, maxq), float32 arithmetic.

    ``w`` is rounded to float32 first (the quantizer's input precision).
    With ``clip=False`` the clamp is omitted (used only for the
    no-clipping condition of Babai's error bound).
    """
    w32 = np.asarray(w, dtype=F64).astype(F32)
    q = np.rint(w32 / np.asarray(s, dtype=F32)).astype(F32) + np.asarray(z, dtype=F32)
    if clip:
        q = np.clip(q, F32(0), F32(maxq))
    return q.astype(F32)


# ---------------------------------------------------------------------------
# a5 + a6: the column sweep.  GPTQ knowledge note, "How It Works": after a
# column is quantized the remaining full-precision columns are adjusted with
# inverse-Hessian information; every row follows one column order; blocks of
# ``block_size`` columns accumulate their corrections before one global
# update of the columns after the block.  With block_size = 1 every update is
# immediate (the unblocked sequential form); any block size gives the same
# result in exact arithmetic.
#
# Column step j (processing order) for every row r:
#   (group start)  (s, z) from the current values of the group's columns
#   c   = clamp(rint(fl32(v_rj / s)) + z, 0, maxq)
#   w^  = s * (c - z)
#   e   = (v_rj - w^) / U_jj
#   v_rk -= e * U_jk   for the later columns k > j   (immediately inside the
#                      block, deferred to the block boundary outside it)
# ---------------------------------------------------------------------------
def gptq_quantize(W, U, perm=None, levels: int = 16, group_size: int = 0,
                  block_size: int = 128, clip: bool = True, order: str = "right",
                  record_inputs: bool = False, forced=None):
    """Quantize W (m x n) with the inverse-Hessian factor U (processing order).

    Returns a dict with (all in processing order unless noted):
      codes   m x n float32 integer-valued codes
      scales  m x G float32, zeros m x G float32 (G groups in processing order)
      E       m x n float64 scaled errors e
      row_loss m float64 = sum_j e_rj^2 / 2
      qin     m x n float64 value each entry had when it was quantized
              (only with record_inputs=True)
    ``order`` selects where the deferred block update is applied:
    "right" after each block to all later columns, "left" to each block just
    before it is swept (identical in exact arithmetic).
    ``forced`` maps (row, column) in processing order to a code that replaces
    the rounding decision there (the rest of the step is unchanged): at a
    rounding tie either code is a correct result, and this follows the other
    branch.
    """
    W = np.asarray(W, dtype=F64)
    U = np.asarray(U, dtype=F64)
    m, n = W.shape
    maxq = int(levels) - 1
    if maxq < 1:
        raise ValueError("levels must be >= 2")
    perm = np.arange(n) if perm is None else np.asarray(perm, dtype=np.int64)
    g = int(group_size)
    if g < 0:
        raise ValueError("group_size must be >= 0")
    B = max(1, int(block_size))
    if B > 1 and g > 0 and B % g != 0 and g % B != 0:
        raise ValueError("blocked sweep needs block_size % group_size == 0 or group_size % block_size == 0")
    if order not in ("right", "left"):
        raise ValueError("order must be 'right' or 'left'")
    G = 1 if g == 0 else -(-n // g)

    V = W[:, perm].copy()
    codes = np.zeros((m, n), dtype=F32)
    E = np.zeros((m, n), dtype=F64)
    scales = np.zeros((m, G), dtype=F32)
    zeros = np.zeros((m, G), dtype=F32)
    qin = np.zeros((m, n), dtype=F64) if record_inputs else None

    if g == 0 and n > 0:
        # Per-row grid: taken from the original row, before any update.
        s_row, z_row = grid_params(V.astype(F32), maxq)
        scales[:, 0], zeros[:, 0] = s_row, z_row
    s_cur = scales[:, 0].copy()
    z_cur = zeros[:, 0].copy()

    # Left-looking order: applied[k] = how many leading columns' errors column
    # k has received.  A group wider than the block takes its statistics from
    # the current values of all its columns, so at its first block every
    # column of the group is brought up to date (right-looking order keeps
    # every later column up to date at each block boundary anyway).
    applied = np.zeros(n, dtype=np.int64)
    for b0 in range(0, n, B):
        b1 = min(n, b0 + B)
        if order == "left" and b0 > 0:
            hi = min(n, b0 + g) if (g > B and b0 % g == 0) else b1
            k0 = int(applied[b0])
            V[:, b0:hi] -= E[:, k0:b0] @ U[k0:b0, b0:hi]
            applied[b0:hi] = b0
        for j in range(b0, b1):
            if g > 0 and j % g == 0:
                gi = j // g
                s_cur, z_cur = grid_params(V[:, j:min(n, j + g)].astype(F32), maxq)
                scales[:, gi], zeros[:, gi] = s_cur, z_cur
            v = V[:, j]
            if record_inputs:
                qin[:, j] = v
            c = quantize_values(v, s_cur, z_cur, maxq, clip=clip)
            if forced:
                for (fr, fj), fc in forced.items():
                    if fj == j:
                        c[fr] = F32(fc)
            what = s_cur.astype(F64) * (c.astype(F64) - z_cur.astype(F64))
            e = (v - what) / U[j, j]
            codes[:, j] = c
            E[:, j] = e
            if j + 1 < b1:
                V[:, j + 1:b1] -= np.outer(e, U[j, j + 1:b1])
        if order == "right" and b1 < n:
            V[:, b1:] -= E[:, b0:b1] @ U[b0:b1, b1:]

    out = dict(codes=codes, scales=scales, zeros=zeros, E=E,
               row_loss=0.5 * np.sum(E * E, axis=1), perm=perm,
               levels=int(levels), group_size=g)
    if record_inputs:
        out["qin"] = qin
    return out


def rtn_quantize(W, levels: int = 16, group_size: int = 0, perm=None):
    """Round-to-nearest on the same grid rule, no error propagation.

    Groups are taken in processing order (``perm``), like the GPTQ sweep.
    Returns the same dict layout as ``gptq_quantize`` (without E/row_loss).
    """
    W = np.asarray(W, dtype=F64)
    m, n = W.shape
    maxq = int(levels) - 1
    perm = np.arange(n) if perm is None else np.asarray(perm, dtype=np.int64)
    V = W[:, perm]
    g = int(group_size)
    G = 1 if g == 0 else -(-n // g)
    codes = np.zeros((m, n), dtype=F32)
    scales = np.zeros((m, G), dtype=F32)
    zeros = np.zeros((m, G), dtype=F32)
    for gi in range(G):
        j0, j1 = (0, n) if g == 0 else (gi * g, min(n, (gi + 1) * g))
        s, z = grid_params(V[:, j0:j1].astype(F32), maxq)
        scales[:, gi], zeros[:, gi] = s, z
        for j in range(j0, j1):
            codes[:, j] = quantize_values(V[:, j], s, z, maxq)
    return dict(codes=codes, scales=scales, zeros=zeros, perm=perm,
                levels=int(levels), group_size=g)


# ---------------------------------------------------------------------------
# a7: outputs in the original column order, packing.
# ---------------------------------------------------------------------------
def unpermute_codes(codes_proc, perm) -> np.ndarray:
    """codes[:, perm[j]] = codes_proc[:, j]."""
    codes_proc = np.asarray(codes_proc)
    out = np.empty_like(codes_proc)
    out[:, np.asarray(perm, dtype=np.int64)] = codes_proc
    return out


def group_index(perm, group_size: int) -> np.ndarray:
    """g_idx[perm[j]] = j // group_size (0 everywhere for per-row grids)."""
    perm = np.asarray(perm, dtype=np.int64)
    n = perm.size
    gidx = np.zeros(n, dtype=np.int32)
    if group_size > 0:
        gidx[perm] = (np.arange(n) // group_size).astype(np.int32)
    return gidx


def dequantize(res) -> np.ndarray:
    """W^ in the original column order, float64: s_g * (c - z_g)."""
    codes = res["codes"].astype(F64)
    m, n = codes.shape
    g = res["group_size"]
    gi = np.zeros(n, dtype=np.int64) if g == 0 else np.arange(n) // g
    s = res["scales"].astype(F64)[:, gi]
    z = res["zeros"].astype(F64)[:, gi]
    return unpermute_codes(s * (codes - z), res["perm"])


def layer_loss(W, What, H) -> float:
    """||(W - W^) X||_F^2 = tr(D (H/2) D^T) with H = 2 X X^T (undamped)."""
    D = np.asarray(W, dtype=F64) - np.asarray(What, dtype=F64)
    return float(np.sum((D @ (0.5 * np.asarray(H, dtype=F64))) * D))


def obs_loss(W, What, Hd, perm) -> np.ndarray:
    """Per-row 1/2 D H_d D^T in processing order (H_d is the damped, permuted H)."""
    perm = np.asarray(perm, dtype=np.int64)
    D = (np.asarray(W, dtype=F64) - np.asarray(What, dtype=F64))[:, perm]
    return 0.5 * np.sum((D @ np.asarray(Hd, dtype=F64)) * D, axis=1)


def packed_words_per_row(n: int, bits: int) -> int:
    return -(-(int(n) * int(bits)) // 32)


def pack_codes(codes, bits: int) -> np.ndarray:
    """Pack b-bit codes row-wise, LSB first, into uint32 words.

    Code k of a row occupies bits [k*b, (k+1)*b) of the row's little-endian
    bit stream (the pages fix no layout; GPTQ knowledge note, "Common
    Confusions": GPTQ is not itself a bit encoding).
    """
    codes = np.asarray(codes, dtype=np.int64)
    m, n = codes.shape
    nw = packed_words_per_row(n, bits)
    out = np.zeros((m, nw), dtype=np.uint64)
    for k in range(n):
        bit = k * bits
        w, off = divmod(bit, 32)
        v = codes[:, k].astype(np.uint64)
        out[:, w] |= (v << np.uint64(off)) & np.uint64(0xFFFFFFFF)
        if off + bits > 32:
            out[:, w + 1] |= v >> np.uint64(32 - off)
    return out.astype(np.uint32)


def unpack_codes(packed, n: int, bits: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint64)
    m = packed.shape[0]
    out = np.zeros((m, n), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for k in range(n):
        bit = k * bits
        w, off = divmod(bit, 32)
        v = packed[:, w] >> np.uint64(off)
        if off + bits > 32:
            v |= packed[:, w + 1] << np.uint64(32 - off)
        out[:, k] = (v & mask).astype(np.int64)
    return out


# ---------------------------------------------------------------------------
# f3: asymmetric calibration (GPTAQ / GPTQv2 abstract on the Daily Papers page
# and the mlsanity page: the quantized layer's output, computed on the
# quantized model's inputs Xq, is matched to the full-precision layer's output
# on the full-precision inputs Xf).  The pages print no closed form.  Reading
# taken (a derivation, not the paper's algorithm): with
#   W' = argmin_V ||Xq V^T - Xf W^T||_F^2 = W Xf^T Xq (Xq^T Xq)^{-1}
# every Q satisfies ||Xq Q^T - Xf W^T||^2 = ||Xq (Q - W')^T||^2 + const
# (Xq W'^T is the projection of Xf W^T onto the column space of Xq), so the
# objective is GPTQ's with H = 2 Xq^T Xq applied to the target W'.  The
# inverse carries GPTQ's own damping: W' = W Hc^T H_d^{-1}, Hc = 2 Xq^T Xf,
# H_d = H + lambda I, which makes W' the ridge solution with penalty
# (lambda/2) ||V||^2.
# ---------------------------------------------------------------------------
def asymmetric_target_from_hessians(W, H, Hc, damp_rel: float) -> np.ndarray:
    """W' = W Hc^T (H + lambda I)^{-1} with lambda = damp_rel mean(diag H), float64."""
    H = np.asarray(H, dtype=F64)
    lam = damp_rel * float(np.mean(np.diag(H)))
    G = np.asarray(W, dtype=F64) @ np.asarray(Hc, dtype=F64).T
    return np.linalg.solve(H + lam * np.eye(H.shape[0]), G.T).T


def asymmetric_target(W, Xq, Xf, damp_rel: float) -> np.ndarray:
    """W' from the inputs: H = 2 Xq^T Xq, Hc = 2 Xq^T Xf (original column order)."""
    Xq = np.asarray(Xq, dtype=F64)
    Xf = np.asarray(Xf, dtype=F64)
    return asymmetric_target_from_hessians(W, 2.0 * (Xq.T @ Xq), 2.0 * (Xq.T @ Xf), damp_rel)


def gptaq_layer(W, Xq, Xf, levels: int = 16, group_size: int = 0, block_size: int = 128,
                damp_rel: float = 0.01, act_order: bool = False):
    """GPTQ with H = 2 Xq^T Xq on the target W' (asymmetric_target)."""
    H = hessian(Xq)
    perm = act_order_perm(H) if act_order else np.arange(H.shape[0])
    Hd, lam = damp_and_permute(H, perm, damp_rel)
    U = inverse_cholesky_upper(Hd)
    Wt = asymmetric_target(W, Xq, Xf, damp_rel)
    res = gptq_quantize(Wt, U, perm, levels, group_size, block_size)
    res.update(Wt=Wt, H=H, Hd=Hd, lam=lam, U=U)
    return res


# ---------------------------------------------------------------------------
# f2: reading the packed weights back (GPTQ knowledge note, "Tradeoffs": the
# speed of a quantized model rests on kernels that consume packed weights,
# inference being limited by weight memory traffic; anthology record
# SOTA-185, "The scope worth holding onto": decode is bandwidth-bound).
# ---------------------------------------------------------------------------
def dequantize_packed(packed, n: int, bits: int, scales, zeros, g_idx) -> np.ndarray:
    """W^[r, k] = s[r, g_idx[k]] * (c[r, k] - z[r, g_idx[k]]), float64.

    ``packed`` is the row-wise LSB-first bit stream of pack_codes (original
    column order); ``g_idx`` gives each original column's group.
    """
    codes = unpack_codes(packed, n, bits).astype(F64)
    gi = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scales, dtype=F64)[:, gi]
    z = np.asarray(zeros, dtype=F64)[:, gi]
    return s * (codes - z)


def dequant_matmul(packed, n: int, bits: int, scales, zeros, g_idx, X) -> np.ndarray:
    """Y = X W^T (batch x m), float64, W^ from dequantize_packed."""
    What = dequantize_packed(packed, n, bits, scales, zeros, g_idx)
    return np.asarray(X, dtype=F64) @ What.T


def dequant_matmul_bound(packed, n: int, bits: int, scales, zeros, g_idx, X) -> np.ndarray:
    """M[b, r] = sum_k s[r, g_k] (c[r, k] + z[r, g_k]) |X[b, k]|, float64.

    The scale of the rounding error of any float32 evaluation of
    dequant_matmul that forms s * (sum c x - z sum x) or sum s (c - z) x.
    """
    codes = unpack_codes(packed, n, bits).astype(F64)
    gi = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scales, dtype=F64)[:, gi]
    z = np.asarray(zeros, dtype=F64)[:, gi]
    return np.abs(np.asarray(X, dtype=F64)) @ (s * (codes + z)).T


# ---------------------------------------------------------------------------
# f4: low-rank correction folded into the GPTQ pass (Daily Papers page,
# GPTQ-intrinsic LoRA abstract): the weights are approximated as Q + L R and
# judged by the layer-wise objective ||X W - X (Q + L R)||_F^2 (there W is
# in x out; here W is out x in, so the correction of W is (L R)^T, L n x r,
# R r x m), with the choice L = V_r, the top-r right singular vectors of X.
# The page names a Hessian augmentation but prints no formula.  Reading taken
# (a derivation from the stated objective): for a fixed L the objective is a
# least-squares problem in R whose minimiser is
#   R* = M^{-1} L^T H (W - Q)^T,  M = L^T H L,  H = 2 X^T X,
# and substituting R* leaves, for every Q,
#   ||(W - Q - R*^T L^T) X^T||^2 = 1/2 tr(D H_L D^T),  D = W - Q,
#   H_L = H - H L M^{-1} L^T H,
# so the GPTQ pass runs unchanged (act-order, damping, U, sweep) on H_L and R*
# is formed from its result.  With L = V_r, H_L = 2 (X - X_r)^T (X - X_r):
# the rank-r residual that replaces ||X||_F^2 in the page's error bound.
# H_L depends on L only through its column span.
# ---------------------------------------------------------------------------
def lowrank_basis(H, r: int) -> np.ndarray:
    """V_r: eigenvectors of H for its r largest eigenvalues (n x r, float64).

    H = 2 X^T X, so these are the top-r right singular vectors of X.
    """
    H = np.asarray(H, dtype=F64)
    if r == 0:
        return np.zeros((H.shape[0], 0), dtype=F64)
    w, V = np.linalg.eigh(H)
    return V[:, np.argsort(w)[::-1][:r]]


def lowrank_hessian(H, L):
    """(H_L, K): H_L = H - H L M^{-1} L^T H and K = H L M^{-1}, M = L^T H L."""
    H = np.asarray(H, dtype=F64)
    L = np.asarray(L, dtype=F64)
    if L.shape[1] == 0:
        return H.copy(), np.zeros((H.shape[0], 0), dtype=F64)
    HL = H @ L
    M = L.T @ HL
    K = np.linalg.solve(M, HL.T).T
    return H - K @ HL.T, K


def lowrank_compensation(W, What, K) -> np.ndarray:
    """R* = K^T (W - W^)^T (r x m): the least-squares R for the quantized W^."""
    D = np.asarray(W, dtype=F64) - np.asarray(What, dtype=F64)
    return (D @ np.asarray(K, dtype=F64)).T


def gptq_lora_layer(W, X=None, H=None, rank: int = 16, levels: int = 16, group_size: int = 0,
                    block_size: int = 128, damp_rel: float = 0.01, act_order: bool = False, L=None,
                    hl_float32: bool = False):
    """GPTQ on the augmented Hessian H_L with L = V_r (or the given L), then R*.

    hl_float32 rounds H_L to float32 before the GPTQ pass, the precision in
    which a float32 Hessian interface hands it on (act-order then sorts the
    same numbers on both sides of such an interface).
    Returns gptq_layer's dictionary for H_L plus H (the undamped calibration
    Hessian), L, K, R and loss_joint = 1/2 tr(D H D^T) with D = W - W^ - R^T L^T.
    """
    W = np.asarray(W, dtype=F64)
    if H is None:
        H = hessian(X)
    H = np.asarray(H, dtype=F64)
    if L is None:
        L = lowrank_basis(H, rank)
    HL, K = lowrank_hessian(H, L)
    if hl_float32:
        HL = HL.astype(F32).astype(F64)
    res = gptq_layer(W, H=HL, levels=levels, group_size=group_size, block_size=block_size,
                     damp_rel=damp_rel, act_order=act_order)
    R = lowrank_compensation(W, res["What"], K)
    D = W - res["What"] - R.T @ np.asarray(L, dtype=F64).T
    res.update(H_aug=res["H"], H=H, L=np.asarray(L, dtype=F64), K=K, R=R,
               loss_joint=0.5 * float(np.sum((D @ H) * D)))
    return res


# ---------------------------------------------------------------------------
# f4 refinement: the Daily Papers page's GPTQ-intrinsic LoRA abstract names
# "Bid-Up", a refinement of the codes on a fixed grid that can alternate with
# the optimal low-rank compensation and never increases the layer-wise
# reconstruction error; it prints no algorithm.  Reading taken (the plainest
# step with that guarantee): cyclic coordinate descent on the codes, with the
# scales, zeros and the current correction C = (L R)^T held fixed.
#
# Row i's error is f(d) = 1/2 d H d^T = ||X d^T||^2 with d = W_i - C_i - W^_i
# and H = 2 X^T X (the undamped calibration Hessian).  Moving the value of
# column j by delta changes f by -delta g_j + delta^2 H_jj / 2 with g = H d,
# so among the grid values s (c - z) of that column the best is the one
# nearest to W^_ij + g_j / H_jj; a move is made only when it lowers f (a tie
# keeps the current code, and a column with H_jj = 0 does not take part), so
# f never increases.  Columns are visited in their original order, rows are
# independent.  Float64 throughout, decisions included (the refinement has no
# float32 interface to reproduce).
#
# Two alternations are offered.  Literal: the refinement with the current R
# fixed, then R = R*.  Joint: since min over R of the joint error is
# 1/2 d H_L d^T with d = W - W^ (H_L = H - H L M^{-1} L^T H), the same
# coordinate descent run on H_L with no correction makes every move optimal
# over the code and R together; R = R* afterwards gives the R it implies.
# Both never increase the joint error.  Where the correction removes strong
# directions of X (H_jj >> (H_L)_jj), the literal step g_j / H_jj seldom
# reaches half a grid step, and the joint one is the one that moves codes.
# ---------------------------------------------------------------------------
def _grid_of_columns(scales, zeros, g_idx, n):
    """Per-element scale and zero (m x n float64) of the fixed grid."""
    gi = np.zeros(n, dtype=np.int64) if g_idx is None else np.asarray(g_idx, dtype=np.int64)
    S = np.asarray(scales, dtype=F32).astype(F64)
    Z = np.asarray(zeros).astype(F64)
    if S.ndim == 1:
        S, Z = S[:, None], Z[:, None]
    return S[:, gi], Z[:, gi]


def refine_codes(W, H, codes, scales, zeros, g_idx, levels: int, sweeps: int = 1, L=None, R=None):
    """Coordinate-descent refinement of the codes on their fixed grid.

    W m x n, H n x n (undamped), codes m x n in original column order, scales
    and zeros m x G, g_idx the group of each column (None: one group per
    row).  L (n x r) and R (r x m) give the low-rank correction held fixed
    (None: no correction).  Returns (codes as int64, moves made in each sweep).
    """
    W = np.asarray(W, dtype=F64)
    H = np.asarray(H, dtype=F64)
    m, n = W.shape
    T = W.copy()
    if L is not None and np.asarray(L).shape[1] > 0:
        T = T - np.asarray(R, dtype=F64).T @ np.asarray(L, dtype=F64).T
    c = np.asarray(codes, dtype=np.int64).copy()
    S, Z = _grid_of_columns(scales, zeros, g_idx, n)
    maxq = levels - 1
    moves = []
    for _ in range(sweeps):
        count = 0
        for i in range(m):
            what = S[i] * (c[i] - Z[i])
            d = T[i] - what
            g = H @ d
            for j in range(n):
                hjj = H[j, j]
                if not hjj > 0:
                    continue
                v = what[j] + g[j] / hjj
                cj = int(min(max(np.rint(v / S[i, j]) + Z[i, j], 0.0), float(maxq)))
                if cj == c[i, j]:
                    continue
                delta = S[i, j] * (cj - Z[i, j]) - what[j]
                gain = delta * g[j] - 0.5 * delta * delta * hjj
                if not gain > 0:
                    continue
                c[i, j] = cj
                what[j] = S[i, j] * (cj - Z[i, j])
                d[j] -= delta
                g -= delta * H[:, j]
                count += 1
        moves.append(count)
    return c, moves


def lora_refine(W, H, L, codes, scales, zeros, g_idx, levels: int, rounds: int = 1, sweeps: int = 1,
                joint: bool = True, HL=None):
    """Alternates the refinement with the compensation R = R*(codes).

    joint=False: the refinement holds the current R fixed (error
    1/2 d H d^T with d = W - W^ - R^T L^T), the literal alternation.
    joint=True: the refinement lowers min over R of the joint error, which
    is 1/2 d H_L d^T with d = W - W^ (the identity behind the low-rank
    path), i.e. the same coordinate descent with H_L and no correction:
    every move is then optimal over the code and R together.  HL overrides
    the H_L formed here (e.g. the float32 H_L another side hands on).
    Both never increase the joint error.  Starts from R*(codes).  Returns
    (codes, R, joint errors 1/2 tr(D H D^T), D = W - W^ - R^T L^T, before
    the first round and after each round).
    """
    W = np.asarray(W, dtype=F64)
    H = np.asarray(H, dtype=F64)
    L = np.asarray(L, dtype=F64)
    HL_formed, K = lowrank_hessian(H, L)
    HL = HL_formed if HL is None else np.asarray(HL, dtype=F64)
    S, Z = _grid_of_columns(scales, zeros, g_idx, W.shape[1])
    c = np.asarray(codes, dtype=np.int64).copy()

    def joint_error(cc, R):
        D = W - S * (cc - Z) - R.T @ L.T
        return 0.5 * float(np.sum((D @ H) * D))

    R = lowrank_compensation(W, S * (c - Z), K)
    losses = [joint_error(c, R)]
    for _ in range(rounds):
        if joint:
            c, _ = refine_codes(W, HL, c, scales, zeros, g_idx, levels, sweeps)
        else:
            c, _ = refine_codes(W, H, c, scales, zeros, g_idx, levels, sweeps, L=L, R=R)
        R = lowrank_compensation(W, S * (c - Z), K)
        losses.append(joint_error(c, R))
    return c, R, losses


# ---------------------------------------------------------------------------
# End to end for one layer.
# ---------------------------------------------------------------------------
def gptq_layer(W, X=None, H=None, levels: int = 16, group_size: int = 0,
               block_size: int = 128, damp_rel: float = 0.01,
               act_order: bool = False, alpha: float = 2.0):
    """Quantize one linear layer: H, damp/permute, U, sweep, outputs.

    Pass either calibration inputs X (tokens x n) or a precomputed H.
    """
    W = np.asarray(W, dtype=F64)
    if H is None:
        H = hessian(X, alpha)
    H = np.asarray(H, dtype=F64)
    perm = act_order_perm(H) if act_order else np.arange(W.shape[1])
    Hd, lam = damp_and_permute(H, perm, damp_rel)
    U = inverse_cholesky_upper(Hd)
    res = gptq_quantize(W, U, perm, levels, group_size, block_size)
    What = dequantize(res)
    bits = max(1, int(np.ceil(np.log2(levels))))
    codes_orig = unpermute_codes(res["codes"], perm).astype(np.int64)
    res.update(H=H, Hd=Hd, lam=lam, U=U, What=What, codes_orig=codes_orig,
               g_idx=group_index(perm, group_size),
               packed=pack_codes(codes_orig, bits), bits=bits,
               loss=layer_loss(W, What, H))
    return res
