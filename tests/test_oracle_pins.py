"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compare the oracle with itself: each checks it against a
hand-worked fixture, a closed form, a textbook algorithm implemented here
independently (Babai's nearest plane algorithm, conditional least squares,
brute-force enumeration, finite differences) or an exact identity.
"""
import inspect
import itertools
import textwrap

import numpy as np
import pytest

import oracle
from oracle import gptq_oracle as go
from tests.conftest import read_golden

F32 = np.float32


def _rng(seed):
    return np.random.default_rng(seed)


def _random_spd(n, rng, cond_mix=0.5, tokens=None):
    tokens = tokens or 4 * n
    X = rng.standard_normal((tokens, n)) @ (np.eye(n) + cond_mix * rng.standard_normal((n, n)))
    return 2.0 * X.T @ X / tokens, X


# ---------------------------------------------------------------------------
# a1 Hessian: H = 2 X X^T is the Hessian of the layer-output loss
# (GPTQ knowledge note, "How It Works").  Pinned by finite differences of
# the loss ||w X||^2, which never forms X^T X.
# ---------------------------------------------------------------------------
def test_hessian_is_second_derivative_of_reconstruction_loss():
    rng = _rng(1)
    N, n = 37, 6
    X = rng.standard_normal((N, n))          # tokens x features
    w0 = rng.standard_normal(n)

    def f(w):
        return float(np.sum((X @ w) ** 2))   # ||w X||^2 in the pages' layout

    h = 0.5
    Hfd = np.zeros((n, n))
    for i in range(n):
        for j in range(n):
            ei, ej = np.eye(n)[i] * h, np.eye(n)[j] * h
            Hfd[i, j] = (f(w0 + ei + ej) - f(w0 + ei) - f(w0 + ej) + f(w0)) / (h * h)
    H = oracle.hessian(X)
    np.testing.assert_allclose(H, Hfd, rtol=1e-10, atol=1e-9)
    # Sampled rows agree with the full matrix.
    np.testing.assert_allclose(oracle.hessian_rows(X, [4, 1], chunk=5), H[[4, 1]], rtol=1e-13)


# ---------------------------------------------------------------------------
# a2 act-order and damping (hand-worked fixture).
# ---------------------------------------------------------------------------
def test_act_order_and_damping_fixture():
    lines = dict(ln.split(None, 1) for ln in read_golden("act_order_damping.txt"))
    d = np.array(lines["perm_diag"].split(), dtype=float)
    expect = np.array(lines["perm_expected"].split(), dtype=int)
    np.testing.assert_array_equal(oracle.act_order_perm(np.diag(d)), expect)

    H = np.diag([1.0, 2.0, 3.0, 4.0])
    H[0, 1] = H[1, 0] = 0.5
    perm = oracle.act_order_perm(H)
    np.testing.assert_array_equal(perm, [3, 2, 1, 0])
    Hd, lam = oracle.damp_and_permute(H, perm, 0.01)
    assert lam == pytest.approx(float(lines["damp_lambda"]), rel=1e-15)
    np.testing.assert_allclose(np.diag(Hd), np.array(lines["damp_diag"].split(), dtype=float), rtol=1e-15)
    assert Hd[2, 3] == Hd[3, 2] == 0.5


def test_act_order_is_stable_descending():
    rng = _rng(2)
    d = rng.integers(0, 5, size=200).astype(float)    # many ties
    perm = oracle.act_order_perm(np.diag(d))
    assert sorted(perm.tolist()) == list(range(200))
    ds = d[perm]
    assert np.all(ds[:-1] >= ds[1:])
    for i in range(199):
        if ds[i] == ds[i + 1]:
            assert perm[i] < perm[i + 1]


# ---------------------------------------------------------------------------
# a3 the inverse factor.  U upper with positive diagonal and U^T U = Hd^-1 is
# unique; pinned against a second route (reverse-order Cholesky of Hd, then a
# triangular inverse) that never forms Hd^-1.
# ---------------------------------------------------------------------------
def test_inverse_factor_two_routes():
    import scipy.linalg as sla
    rng = _rng(3)
    for n in (1, 2, 5, 33, 130):
        Hd, _ = _random_spd(n, rng)
        U = oracle.inverse_cholesky_upper(Hd)
        assert np.allclose(np.tril(U, -1), 0)
        assert np.all(np.diag(U) > 0)
        np.testing.assert_allclose(U.T @ U @ Hd, np.eye(n), atol=1e-9)
        J = np.eye(n)[::-1]
        L = np.linalg.cholesky(J @ Hd @ J)
        R = J @ L @ J                       # Hd = R R^T, R upper
        U2 = sla.solve_triangular(R, np.eye(n), lower=False)
        np.testing.assert_allclose(U, U2, rtol=1e-9, atol=1e-12)


def test_not_positive_definite_reports_pivot():
    H = np.diag([1.0, 2.0, 0.0, 3.0])
    with pytest.raises(oracle.NotPositiveDefinite) as ei:
        oracle.inverse_cholesky_upper(H)
    assert ei.value.index == 3
    with pytest.raises(oracle.NotPositiveDefinite):
        oracle.inverse_cholesky_upper(np.zeros((3, 3)))


# ---------------------------------------------------------------------------
# a4 grid parameters (hand-worked fixture).
# ---------------------------------------------------------------------------
def test_grid_fixture():
    for ln in read_golden("grid_asymmetric.txt"):
        head, vals, sz, codes = [p.strip() for p in ln.split("|")]
        _, levels = head.split()
        levels = int(levels)
        v = np.array(vals.split(), dtype=F32)
        s_exp, z_exp = sz.split()
        s, z = oracle.grid_params(v[None, :], levels - 1)
        assert s[0] == F32(float(s_exp))
        assert z[0] == float(z_exp)
        c = oracle.quantize_values(v, s, z, levels - 1)
        np.testing.assert_array_equal(c, np.array(codes.split(), dtype=F32))


def test_grid_reconstruction_error_bounded():
    rng = _rng(4)
    for levels in (3, 4, 8, 16):
        W = rng.standard_normal((50, 64)) * 0.02
        s, z = oracle.grid_params(W.astype(F32), levels - 1)
        c = oracle.quantize_values(W, s[:, None], z[:, None], levels - 1)
        assert c.min() >= 0 and c.max() <= levels - 1
        what = s[:, None].astype(float) * (c - z[:, None])
        # Inside the range every value is within half a step of its grid point.
        assert np.all(np.abs(W.astype(F32) - what) <= 0.5 * s[:, None] * (1 + 1e-5))


# ---------------------------------------------------------------------------
# a5/a6 the sweep.
# ---------------------------------------------------------------------------
def test_three_column_fixture():
    g = dict(ln.split(None, 1) for ln in read_golden("gptq_three_columns.txt"))
    U = np.array([[float(x) for x in row.split()] for row in g["U"].split("|")])
    w = np.array(g["w"].split(), dtype=F32).astype(float)[None, :]
    levels = int(g["levels"])
    res = oracle.gptq_quantize(w, U, None, levels, 0, block_size=1, record_inputs=True)
    assert res["scales"][0, 0] == F32(float(g["scale"]))
    assert res["zeros"][0, 0] == float(g["zero"])
    np.testing.assert_array_equal(res["codes"][0], np.array(g["codes"].split(), dtype=float))
    assert res["qin"][0, 1] == pytest.approx(float(g["qin1"]), rel=1e-12)
    rtn = oracle.rtn_quantize(w, levels, 0)
    np.testing.assert_array_equal(rtn["codes"][0], np.array(g["rtn_codes"].split(), dtype=float))
    Hd = np.array([[1, 0.9, 0], [0.9, 1, 0], [0, 0, 1.0]])
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(3), atol=1e-12)
    assert res["row_loss"][0] == pytest.approx(float(g["obs_loss"]), rel=1e-6)
    for r, key in ((res, "obs_loss"), (rtn, "rtn_obs_loss")):
        What = oracle.dequantize(r)
        assert oracle.obs_loss(w, What, Hd, np.arange(3))[0] == pytest.approx(float(g[key]), rel=1e-6)


@pytest.mark.parametrize("levels,group,act", [(16, 0, False), (16, 8, True), (8, 16, False),
                                              (4, 0, True), (3, 8, False)])
def test_identity_hessian_reduces_to_rtn(levels, group, act):
    """H = I (any damping): U is diagonal, nothing is propagated, GPTQ = RTN bit for bit."""
    rng = _rng(5)
    m, n = 40, 64
    W = (rng.standard_normal((m, n)) * 0.02).astype(F32).astype(float)
    res = oracle.gptq_layer(W, H=np.eye(n), levels=levels, group_size=group, act_order=act,
                            block_size=16)
    np.testing.assert_array_equal(res["perm"], np.arange(n))     # ties keep natural order
    rtn = oracle.rtn_quantize(W, levels, group)
    np.testing.assert_array_equal(res["codes"], rtn["codes"])
    np.testing.assert_array_equal(res["scales"], rtn["scales"])
    np.testing.assert_array_equal(res["zeros"], rtn["zeros"])
    # Diagonal, non-constant H with act-order: still RTN, in processing-order groups.
    d = rng.uniform(1, 2, size=n)
    res2 = oracle.gptq_layer(W, H=np.diag(d), levels=levels, group_size=group, act_order=act,
                             block_size=16)
    rtn2 = oracle.rtn_quantize(W, levels, group, perm=res2["perm"])
    np.testing.assert_array_equal(res2["codes"], rtn2["codes"])


def _sweep_case(seed, m=7, n=24, levels=16, group=0, act=True, clip=True, block=1, order="right"):
    rng = _rng(seed)
    H, _ = _random_spd(n, rng, cond_mix=0.7)
    W = rng.standard_normal((m, n)) * 0.05
    perm = oracle.act_order_perm(H) if act else np.arange(n)
    Hd, _ = oracle.damp_and_permute(H, perm, 0.01)
    U = oracle.inverse_cholesky_upper(Hd)
    res = oracle.gptq_quantize(W, U, perm, levels, group, block_size=block, clip=clip,
                               order=order, record_inputs=True)
    return W, H, Hd, U, perm, res


@pytest.mark.parametrize("seed,levels,group,act,block", [(10, 16, 0, False, 1), (11, 8, 8, True, 1),
                                                         (12, 4, 4, True, 8), (13, 3, 0, False, 4),
                                                         (14, 16, 8, True, 8)])
def test_conditional_least_squares_definition(seed, levels, group, act, block):
    """The value quantized at step j is the j-th coordinate of
    argmin_v ||w - v||_{Hd} with v_<j fixed to the grid values already chosen.
    Solved directly with a linear solve on Hd; U is never used."""
    W, H, Hd, U, perm, res = _sweep_case(seed, levels=levels, group=group, act=act, block=block)
    V0 = W[:, perm]
    n = V0.shape[1]
    g = res["group_size"]
    gi = np.zeros(n, int) if g == 0 else np.arange(n) // g
    What = res["scales"].astype(float)[:, gi] * (res["codes"] - res["zeros"].astype(float)[:, gi])
    for j in range(n):
        a, b = slice(0, j), slice(j, n)
        dA = V0[:, a] - What[:, a]
        vb = V0[:, b] + np.linalg.solve(Hd[b, b], Hd[b, a] @ dA.T).T
        np.testing.assert_allclose(res["qin"][:, j], vb[:, 0], rtol=1e-9, atol=1e-12)


def test_loss_identity():
    """sum_j e_j^2 / 2 = 1/2 D Hd D^T = ||D X||^2 + lam/2 ||D||^2 (exact, any grid)."""
    rng = _rng(20)
    for trial in range(20):
        n = int(rng.integers(2, 40))
        m = int(rng.integers(1, 9))
        X = rng.standard_normal((3 * n, n)) * np.exp(rng.standard_normal(n))
        W = rng.standard_normal((m, n)) * 0.05
        levels = int(rng.choice([3, 4, 8, 16]))
        group = int(rng.choice([0, 2, 4]))
        act = bool(rng.integers(0, 2))
        res = oracle.gptq_layer(W, X=X, levels=levels, group_size=group, act_order=act, block_size=4)
        D = W - res["What"]
        np.testing.assert_allclose(res["row_loss"], oracle.obs_loss(W, res["What"], res["Hd"], res["perm"]),
                                   rtol=1e-9)
        dx = float(np.sum((D @ X.T) ** 2))
        np.testing.assert_allclose(res["row_loss"].sum(), dx + 0.5 * res["lam"] * np.sum(D * D), rtol=1e-9)
        np.testing.assert_allclose(res["loss"], dx, rtol=1e-9)


def _babai_nearest_plane(t, G):
    """Textbook nearest-plane back-substitution for min_y ||t - y||_G over integers,
    G = R^T R with R upper (Cholesky of G): y_j = rint(t_j + sum_{k>j} R_jk (t_k - y_k) / R_jj)."""
    R = np.linalg.cholesky(G).T
    n = t.size
    y = np.zeros(n)
    for j in range(n - 1, -1, -1):
        y[j] = np.rint(t[j] + np.dot(R[j, j + 1:], t[j + 1:] - y[j + 1:]) / R[j, j])
    return y


def test_back_to_front_gptq_is_babai_nearest_plane():
    """Daily Papers page, abstract on GPTQ and Babai's nearest plane algorithm:
    run back to front with no clipping, GPTQ equals nearest plane on the lattice of
    the Hessian.  Grid coordinates: t = w / s, integer y = code - zero."""
    rng = _rng(30)
    mism = 0
    total = 0
    for trial in range(400):
        n = int(rng.integers(3, 7))
        H, _ = _random_spd(n, rng, cond_mix=1.0)
        w = rng.standard_normal((1, n)) * 0.05
        back = np.arange(n)[::-1]
        Hd, _ = oracle.damp_and_permute(H, back, 0.01)
        U = oracle.inverse_cholesky_upper(Hd)
        res = oracle.gptq_quantize(w, U, back, 16, 0, block_size=1, clip=False)
        s, z = res["scales"][0, 0], res["zeros"][0, 0]
        y_gptq = oracle.unpermute_codes(res["codes"], back)[0] - z
        Hd_nat, _ = oracle.damp_and_permute(H, None, 0.01)
        t = w[0].astype(F32).astype(float) / float(s)
        y_babai = _babai_nearest_plane(t, Hd_nat)
        mism += int(np.sum(y_gptq != y_babai))
        total += n
    assert mism == 0, f"{mism} of {total} coordinates differ"


def test_babai_error_bound_and_brute_force_optimum():
    """No clipping: ||D||^2_{Hd} <= (s^2/4) sum_j U_jj^-2 (Babai's bound).
    2-bit, n <= 6: the grid optimum found by enumeration is never above the
    oracle's loss, and the loss of the oracle's codes evaluated directly
    equals the reported loss."""
    rng = _rng(31)
    for trial in range(150):
        n = int(rng.integers(2, 7))
        H, _ = _random_spd(n, rng, cond_mix=1.0)
        w = rng.standard_normal((1, n)) * 0.05
        Hd, _ = oracle.damp_and_permute(H, None, 0.01)
        U = oracle.inverse_cholesky_upper(Hd)
        res = oracle.gptq_quantize(w, U, None, 4, 0, block_size=1, clip=False)
        s = float(res["scales"][0, 0])
        D = w - oracle.dequantize(res)
        lossH = float((D @ Hd @ D.T)[0, 0])
        assert lossH <= (s * s / 4) * np.sum(np.diag(U) ** -2) * (1 + 1e-9)
        # brute force over the clipped 2-bit grid
        resc = oracle.gptq_quantize(w, U, None, 4, 0, block_size=1, clip=True)
        z = float(resc["zeros"][0, 0])
        best = np.inf
        for codes in itertools.product(range(4), repeat=n):
            d = w[0] - s * (np.array(codes) - z)
            best = min(best, float(d @ Hd @ d))
        Dc = w - oracle.dequantize(resc)
        mine = float((Dc @ Hd @ Dc.T)[0, 0])
        assert best <= mine * (1 + 1e-12)
        assert 2 * resc["row_loss"][0] == pytest.approx(mine, rel=1e-9)


def test_gptq_not_worse_than_rtn_two_columns():
    """n <= 2: column 0 is RTN and column 1 is the exact 1-D minimiser, so GPTQ's
    loss in the damped metric never exceeds RTN's (provable only for n <= 2)."""
    rng = _rng(32)
    for trial in range(500):
        n = int(rng.integers(1, 3))
        H, _ = _random_spd(n, rng, cond_mix=1.0)
        w = rng.standard_normal((1, n)) * 0.05
        levels = int(rng.choice([3, 4, 8, 16]))
        Hd, _ = oracle.damp_and_permute(H, None, 0.01)
        U = oracle.inverse_cholesky_upper(Hd)
        res = oracle.gptq_quantize(w, U, None, levels, 0, block_size=1)
        rtn = oracle.rtn_quantize(w, levels, 0)
        lg = oracle.obs_loss(w, oracle.dequantize(res), Hd, np.arange(n))[0]
        lr = oracle.obs_loss(w, oracle.dequantize(rtn), Hd, np.arange(n))[0]
        assert lg <= lr * (1 + 1e-12) + 1e-18


@pytest.mark.parametrize("levels,group,act", [(16, 0, False), (8, 16, True), (4, 32, False), (3, 0, True)])
def test_block_size_and_update_order_invariance(levels, group, act):
    """Lazy batching (GPTQ knowledge note, "How It Works": blocks accumulate
    corrections before a global update) changes only rounding order: B = 1,
    right-looking B = 32 and left-looking B = 32 give the same codes."""
    rng = _rng(40)
    n, m = 96, 30
    X = rng.standard_normal((4 * n, n)) @ (np.eye(n) + 0.3 * rng.standard_normal((n, n)))
    W = rng.standard_normal((m, n)) * 0.05
    H = oracle.hessian(X)
    perm = oracle.act_order_perm(H) if act else np.arange(n)
    Hd, _ = oracle.damp_and_permute(H, perm, 0.01)
    U = oracle.inverse_cholesky_upper(Hd)
    r1 = oracle.gptq_quantize(W, U, perm, levels, group, block_size=1)
    r2 = oracle.gptq_quantize(W, U, perm, levels, group, block_size=32, order="right")
    r3 = oracle.gptq_quantize(W, U, perm, levels, group, block_size=32, order="left")
    for r in (r2, r3):
        np.testing.assert_array_equal(r["codes"], r1["codes"])
        np.testing.assert_array_equal(r["scales"], r1["scales"])
        np.testing.assert_allclose(r["E"], r1["E"], rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("levels,group,act", [(16, 64, False), (8, 96, True), (4, 64, True)])
def test_groups_wider_than_the_block(levels, group, act):
    """Groups spanning several blocks take their range from the current values
    of all their columns at the group start: B = 1 (the unblocked definition),
    right-looking B = 32 and left-looking B = 32 agree."""
    rng = _rng(44)
    n, m = 200, 25
    X = rng.standard_normal((4 * n, n)) @ (np.eye(n) + 0.3 * rng.standard_normal((n, n)))
    W = rng.standard_normal((m, n)) * 0.05
    H = oracle.hessian(X)
    perm = oracle.act_order_perm(H) if act else np.arange(n)
    Hd, _ = oracle.damp_and_permute(H, perm, 0.01)
    U = oracle.inverse_cholesky_upper(Hd)
    r1 = oracle.gptq_quantize(W, U, perm, levels, group, block_size=1)
    r2 = oracle.gptq_quantize(W, U, perm, levels, group, block_size=32, order="right")
    r3 = oracle.gptq_quantize(W, U, perm, levels, group, block_size=32, order="left")
    assert r1["scales"].shape[1] == -(-n // group)
    for r in (r2, r3):
        np.testing.assert_array_equal(r["codes"], r1["codes"])
        np.testing.assert_array_equal(r["scales"], r1["scales"])
        np.testing.assert_allclose(r["E"], r1["E"], rtol=1e-9, atol=1e-12)
    # A group statistic taken before the earlier corrections reach the group's
    # later columns would differ: with U diagonal the range of a whole group
    # is that of the original weights (RTN), here it is not.
    rtn = oracle.rtn_quantize(W, levels, group, perm=perm)
    assert not np.array_equal(rtn["scales"][:, 1:], r1["scales"][:, 1:])


def test_hessian_scale_invariance_and_row_independence():
    rng = _rng(41)
    n, m = 48, 20
    X = rng.standard_normal((3 * n, n)) * np.exp(rng.standard_normal(n))
    W = rng.standard_normal((m, n)) * 0.05
    H = oracle.hessian(X)
    a = oracle.gptq_layer(W, H=H, levels=8, group_size=16, act_order=True, block_size=16)
    b = oracle.gptq_layer(W, H=H * 37.0, levels=8, group_size=16, act_order=True, block_size=16)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    rows = [3, 17, 0]
    c = oracle.gptq_quantize(W[rows], a["U"], a["perm"], 8, 16, block_size=16)
    np.testing.assert_array_equal(c["codes"], a["codes"][rows])
    np.testing.assert_array_equal(c["scales"], a["scales"][rows])


def test_outputs_original_order_and_group_index():
    rng = _rng(42)
    n, m = 40, 5
    X = rng.standard_normal((3 * n, n)) * np.exp(rng.standard_normal(n))
    W = rng.standard_normal((m, n)) * 0.05
    res = oracle.gptq_layer(W, X=X, levels=8, group_size=8, act_order=True, block_size=8)
    perm = res["perm"]
    for j in range(n):
        np.testing.assert_array_equal(res["codes_orig"][:, perm[j]], res["codes"][:, j])
        assert res["g_idx"][perm[j]] == j // 8
    # Dequantized weights use the group of each original column.
    s = res["scales"].astype(float)[:, res["g_idx"]]
    z = res["zeros"].astype(float)[:, res["g_idx"]]
    np.testing.assert_allclose(res["What"], s * (res["codes_orig"] - z), rtol=0, atol=0)


# ---------------------------------------------------------------------------
# a7 packing.
# ---------------------------------------------------------------------------
def test_packed_layout_fixture_and_sizes():
    lines = read_golden("packed_layout.txt")
    kv = {}
    for ln in lines:
        if "|" in ln:
            bits, codes, words = [p.strip() for p in ln.split("|")]
            c = np.array([codes.split()], dtype=np.int64)
            w = np.array([[int(x, 16) for x in words.split()]], dtype=np.uint32)
            np.testing.assert_array_equal(oracle.pack_codes(c, int(bits)), w)
            np.testing.assert_array_equal(oracle.unpack_codes(w, c.shape[1], int(bits)), c)
        else:
            k, v = ln.split()
            kv[k] = int(v)
    p = kv["params"]
    assert p * 4 // 8 == kv["bytes_4bit"]
    assert p * 16 // 8 == kv["bytes_16bit"]
    assert kv["bytes_16bit"] // kv["bytes_4bit"] == 4
    assert oracle.packed_words_per_row(p, 4) * 4 == kv["bytes_4bit"]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_round_trip(bits):
    rng = _rng(50 + bits)
    for n in (1, 7, 32, 33, 95, 130):
        c = rng.integers(0, 1 << bits, size=(3, n))
        p = oracle.pack_codes(c, bits)
        assert p.shape == (3, -(-n * bits // 32))
        np.testing.assert_array_equal(oracle.unpack_codes(p, n, bits), c)


# ---------------------------------------------------------------------------
# Planted mistakes: a copy of the oracle's sweep with one plausible error must
# fail at least one of the pins above.
# ---------------------------------------------------------------------------
MUTATIONS = {
    "update sign": ("V[:, j + 1:b1] -= np.outer(e, U[j, j + 1:b1])",
                    "V[:, j + 1:b1] += np.outer(e, U[j, j + 1:b1])"),
    "wrong U row": ("V[:, j + 1:b1] -= np.outer(e, U[j, j + 1:b1])",
                    "V[:, j + 1:b1] -= np.outer(e, U[j + 1:b1, j])"),
    "no diagonal scaling": ("e = (v - what) / U[j, j]", "e = (v - what)"),
    "dropped block update": ("V[:, b1:] -= E[:, b0:b1] @ U[b0:b1, b1:]", "pass"),
    "transposed block update": ("V[:, b1:] -= E[:, b0:b1] @ U[b0:b1, b1:]",
                                "V[:, b1:] -= E[:, b0:b1] @ U[b1:, b0:b1].T"),
}


def _mutated_sweep(old, new):
    src = textwrap.dedent(inspect.getsource(go.gptq_quantize))
    assert old in src
    ns = dict(go.__dict__)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["gptq_quantize"]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    mutant = _mutated_sweep(*MUTATIONS[name])
    monkeypatch.setattr(go, "gptq_quantize", mutant)
    monkeypatch.setattr(oracle, "gptq_quantize", mutant)
    caught = []
    for check in (lambda: test_conditional_least_squares_definition(14, 16, 8, True, 8),
                  test_loss_identity,
                  lambda: test_block_size_and_update_order_invariance(16, 0, False)):
        try:
            check()
        except AssertionError:
            caught.append(check)
    assert caught, f"mutation '{name}' was not caught by any pin"


# ---------------------------------------------------------------------------
# f2 reading the packed weights back.
# ---------------------------------------------------------------------------
def test_dequant_matvec_fixture():
    kv = dict(ln.split(None, 1) for ln in read_golden("dequant_matvec.txt"))
    bits, n = int(kv["bits"]), int(kv["n"])
    g_idx = np.array(kv["g_idx"].split(), dtype=np.int32)
    codes = np.array([kv["codes0"].split(), kv["codes1"].split()], dtype=np.int64)
    words = np.array([[int(kv["word0"], 16)], [int(kv["word1"], 16)]], dtype=np.uint32)
    scales = np.array([kv["scales0"].split(), kv["scales1"].split()], dtype=np.float32)
    zeros = np.array([kv["zeros0"].split(), kv["zeros1"].split()], dtype=np.uint8)
    X = np.array([kv["x0"].split(), kv["x1"].split()], dtype=np.float64)
    Y = np.array([kv["y0"].split(), kv["y1"].split()], dtype=np.float64)
    np.testing.assert_array_equal(oracle.pack_codes(codes, bits), words)
    np.testing.assert_array_equal(oracle.unpack_codes(words, n, bits), codes)
    np.testing.assert_array_equal(oracle.dequant_matmul(words, n, bits, scales, zeros, g_idx, X), Y)


@pytest.mark.parametrize("levels,group,act", [(16, 0, False), (8, 32, True), (4, 64, False), (3, 16, True)])
def test_dequant_packed_matches_the_sweep_dequantization(levels, group, act):
    # Two routes to W^: dequantize() reads the sweep's processing-order codes
    # and groups and un-permutes; dequantize_packed() reads the packed stream
    # in original order and looks each column's group up in g_idx.
    rng = np.random.default_rng(7 + levels + group)
    m, n = 6, 96
    W = rng.normal(0.0, 0.02, size=(m, n))
    X = rng.standard_normal((300, n)) * np.exp(rng.normal(0.0, 1.0, size=n))
    res = oracle.gptq_layer(W, X=X, levels=levels, group_size=group, act_order=act)
    Wp = oracle.dequantize_packed(res["packed"], n, res["bits"], res["scales"], res["zeros"], res["g_idx"])
    np.testing.assert_array_equal(Wp, res["What"])
    xb = rng.standard_normal((3, n))
    np.testing.assert_allclose(oracle.dequant_matmul(res["packed"], n, res["bits"], res["scales"], res["zeros"],
                                                     res["g_idx"], xb), xb @ res["What"].T, rtol=1e-12, atol=1e-15)
    M = oracle.dequant_matmul_bound(res["packed"], n, res["bits"], res["scales"], res["zeros"], res["g_idx"], xb)
    assert np.all(M >= np.abs(xb) @ np.abs(res["What"]).T)


# ---------------------------------------------------------------------------
# f1 whole-decoder pass (oracle.decoder_oracle).
# ---------------------------------------------------------------------------
def test_decoder_pieces_closed_forms():
    D = oracle.decoder_oracle
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 12)) * 3.0
    y = D.rms_norm(x, eps=1e-6)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + 1e-6), rtol=1e-12)
    # RoPE: position 0 is the identity, norms of rotated pairs are kept, and
    # <rope(q) at m, rope(k) at n> depends only on m - n.
    q = rng.standard_normal((1, 6, 2, 8))
    k = rng.standard_normal((1, 6, 2, 8))
    rq, rk = D.rope(np.repeat(q[:, :1], 6, axis=1)), D.rope(np.repeat(k[:, :1], 6, axis=1))
    np.testing.assert_allclose(rq[:, 0], q[:, 0], rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(np.repeat(q[:, :1], 6, axis=1), axis=-1),
                               rtol=1e-12)
    d1 = np.sum(rq[0, 4] * rk[0, 1], axis=-1)
    d2 = np.sum(rq[0, 5] * rk[0, 2], axis=-1)
    np.testing.assert_allclose(d1, d2, rtol=1e-10)
    # Causal attention: position 0 sees only itself (output = v_0); with two
    # positions and q0 = k0 = 0, q1 . k1 = 0, k0 = 0: position 1 averages v0, v1.
    Iq = np.eye(4)
    h = np.array([[1.0, 2.0, 0.0, 0.0], [0.0, 0.0, 3.0, 5.0]])
    Wz = np.zeros((4, 4))
    out = D.attention(h, Wz, Wz, Iq, n_heads=1, seqs=1, seq_len=2)
    np.testing.assert_allclose(out[0], h[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[1], 0.5 * (h[0] + h[1]), rtol=1e-15)


def test_silu_closed_forms():
    # silu(x) = x * sigmoid(x): odd part x / 2, silu(x) - silu(-x) = x, value
    # 0 and slope 1/2 at 0, e/(1 + e) at 1, x for large x, 0 for very negative x.
    D = oracle.decoder_oracle
    x = np.linspace(-6.0, 6.0, 49)
    y = D.silu(x)
    np.testing.assert_allclose(y - D.silu(-x), x, rtol=0, atol=1e-14)
    assert D.silu(np.array(0.0)) == 0.0
    h = 1e-6
    np.testing.assert_allclose((D.silu(np.array(h)) - D.silu(np.array(-h))) / (2 * h), 0.5, rtol=1e-9)
    np.testing.assert_allclose(D.silu(np.array([1.0, -1.0, 2.0])),
                               [np.e / (1 + np.e), -1 / (1 + np.e), 2 * np.e ** 2 / (1 + np.e ** 2)], rtol=1e-15)
    np.testing.assert_allclose(D.silu(np.array(40.0)), 40.0, rtol=1e-15)
    assert abs(float(D.silu(np.array(-40.0)))) < 1e-15
    # gating below the threshold: silu is below the identity for x > 0 and negative for x < 0
    assert np.all(y[x > 0] < x[x > 0]) and np.all(y[x < 0] < 0)


def test_attention_against_explicit_rotations_and_softmax():
    # The oracle's attention against a second formulation: RoPE as explicit
    # 2 x 2 rotation matrices on the pairs (i, i + D/2) with angle
    # p * 10000^(-2i/D), softmax from scipy, causal mask as a loop bound.
    from scipy.special import softmax
    D = oracle.decoder_oracle
    rng = np.random.default_rng(17)
    d, heads, seqs, S = 16, 2, 2, 5
    hd = d // heads
    h = rng.standard_normal((seqs * S, d))
    Wq, Wk, Wv = (rng.standard_normal((d, d)) * 0.3 for _ in range(3))

    def rot(vec, p):
        out = vec.copy()
        for i in range(hd // 2):
            th = p * 10000.0 ** (-2.0 * i / hd)
            R = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
            out[[i, i + hd // 2]] = R @ vec[[i, i + hd // 2]]
        return out

    ref = np.zeros((seqs * S, d))
    for s in range(seqs):
        for t in range(S):
            x_t = h[s * S + t]
            for hh in range(heads):
                sl = slice(hh * hd, (hh + 1) * hd)
                q = rot((Wq @ x_t)[sl], t)
                ks = [rot((Wk @ h[s * S + u])[sl], u) for u in range(t + 1)]
                vs = [(Wv @ h[s * S + u])[sl] for u in range(t + 1)]
                p_ = softmax(np.array([q @ k for k in ks]) / np.sqrt(hd))
                ref[s * S + t, sl] = sum(pi * v for pi, v in zip(p_, vs))
    np.testing.assert_allclose(D.attention(h, Wq, Wk, Wv, heads, seqs, S), ref, rtol=1e-12, atol=1e-13)


def test_rms_norm_by_hand():
    D = oracle.decoder_oracle
    x = np.array([[3.0, 4.0], [1.0, -1.0]])
    # mean squares 12.5 and 1
    np.testing.assert_allclose(D.rms_norm(x, eps=0.0), [[3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], [1.0, -1.0]],
                               rtol=1e-15)


def _silu_ref(x):
    from scipy.special import expit
    return x * expit(x)


def _forward_inputs(blocks_what, X, n_heads, seqs, seq_len):
    """Layer inputs of every block recomputed token-block by token-block from
    the final (dequantized) weights -- a second, independent formulation of
    which activations each layer sees."""
    D = oracle.decoder_oracle
    inputs = []
    for W in blocks_what:
        h = D.rms_norm(X)
        parts = [D.attention(h[s * seq_len:(s + 1) * seq_len], W["q"], W["k"], W["v"], n_heads, 1, seq_len)
                 for s in range(seqs)]
        a = np.concatenate(parts, axis=0)
        X = X + a @ W["o"].T
        h2 = D.rms_norm(X)
        mm = _silu_ref(h2 @ W["gate"].T) * (h2 @ W["up"].T)
        X = X + mm @ W["down"].T
        inputs.append(dict(q=h, k=h, v=h, o=a, gate=h2, up=h2, down=mm))
    return X, inputs


@pytest.mark.parametrize("levels,group,act", [(4, 32, False), (3, 0, True)])
def test_decoder_pass_feeds_each_layer_the_quantized_predecessors(levels, group, act):
    # The loss identity sum_j e_rj^2/2 = 1/2 (w - w^) H_d (w - w^)^T holds for
    # each layer exactly when its Hessian was formed from the inputs the
    # sequential protocol defines (quantized earlier layers).
    D = oracle.decoder_oracle
    rng = np.random.default_rng(11 + levels)
    d, f, heads, nb, seqs, S = 32, 64, 2, 2, 3, 16
    blocks = [{k: (rng.standard_normal(shp) * 0.1).astype(np.float32)
               for k, shp in dict(q=(d, d), k=(d, d), v=(d, d), o=(d, d), gate=(f, d), up=(f, d), down=(d, f)).items()}
              for _ in range(nb)]
    X0 = rng.standard_normal((seqs * S, d))
    Xo, res = D.quantize_decoder(blocks, X0, heads, seqs, S, levels=levels, group_size=group, act_order=act)
    Xr, inputs = _forward_inputs([{k: r[k]["What"] for k in r} for r in res], X0, heads, seqs, S)
    np.testing.assert_allclose(Xo, Xr, rtol=1e-10, atol=1e-12)
    for b in range(nb):
        assert np.array_equal(res[b]["q"]["perm"], res[b]["k"]["perm"])
        assert np.array_equal(res[b]["gate"]["perm"], res[b]["up"]["perm"])
        for name, r in res[b].items():
            H = oracle.hessian(inputs[b][name].astype(np.float32).astype(np.float64))
            Hd, _ = oracle.damp_and_permute(H, r["perm"], 0.01)
            np.testing.assert_allclose(oracle.obs_loss(r["W"], r["What"], Hd, r["perm"]), r["row_loss"], rtol=1e-7)


# ---------------------------------------------------------------------------
# f3 asymmetric calibration target.
# ---------------------------------------------------------------------------
def test_asymmetric_target_properties():
    rng = np.random.default_rng(21)
    T, n, m = 400, 24, 7
    W = rng.standard_normal((m, n))
    Xf = rng.standard_normal((T, n)) * np.exp(rng.normal(0, 0.5, size=n))
    Xq = Xf + 0.05 * rng.standard_normal((T, n))
    # Same inputs, no damping: the target is W itself.
    np.testing.assert_allclose(oracle.asymmetric_target(W, Xf, Xf, 0.0), W, rtol=1e-9, atol=1e-11)
    # No damping: ||Xq Q^T - Xf W^T||^2 = ||Xq (Q - W')^T||^2 + ||Xq W'^T - Xf W^T||^2 for any Q.
    Wt = oracle.asymmetric_target(W, Xq, Xf, 0.0)
    Q = np.round(W * 3) / 3
    lhs = np.sum((Xq @ Q.T - Xf @ W.T) ** 2)
    rhs = np.sum((Xq @ (Q - Wt).T) ** 2) + np.sum((Xq @ Wt.T - Xf @ W.T) ** 2)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10)
    # Damped: W' is the ridge solution, Xq^T (Xq W'^T - Xf W^T) + (lambda/2) W'^T = 0.
    damp = 0.01
    Wd = oracle.asymmetric_target(W, Xq, Xf, damp)
    lam = damp * np.mean(np.diag(2 * Xq.T @ Xq))
    grad = Xq.T @ (Xq @ Wd.T - Xf @ W.T) + 0.5 * lam * Wd.T
    assert np.max(np.abs(grad)) <= 1e-9 * np.max(np.abs(Xq.T @ Xf @ W.T))


def test_gptaq_reduces_to_gptq_on_symmetric_inputs():
    rng = np.random.default_rng(22)
    W = rng.normal(0, 0.02, size=(5, 40))
    X = rng.standard_normal((300, 40)) * np.exp(rng.normal(0, 1.0, size=40))
    a = oracle.gptaq_layer(W, X, X, levels=8, group_size=0, damp_rel=0.0, act_order=True)
    b = oracle.gptq_layer(W, X=X, levels=8, group_size=0, damp_rel=0.0, act_order=True)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_allclose(a["Wt"], W, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------------------
# f4 low-rank correction (GPTQ-intrinsic LoRA abstract, Daily Papers page).
# Pinned without the closed forms: for every code vector on a small grid the
# joint optimum over R is found by a least-squares solve on X L (H_L is never
# formed), and L = V_r against a truncated SVD of X.
# ---------------------------------------------------------------------------
def _lora_inputs(seed, T=40, n=5, m=3, spikes=(6.0, 3.0)):
    rng = _rng(seed)
    X = rng.standard_normal((T, n))
    for s in spikes:
        X += s * np.outer(rng.standard_normal(T), rng.standard_normal(n)) / np.sqrt(n)
    return X, rng.standard_normal((m, n)), rng


def test_lowrank_hessian_is_the_joint_optimum_over_r():
    X, W, rng = _lora_inputs(31)
    n = X.shape[1]
    H = 2.0 * X.T @ X
    for r in (1, 2):
        Ls = (oracle.lowrank_basis(H, r), np.linalg.qr(rng.standard_normal((n, r)))[0])
        for L in Ls:
            HL, K = oracle.lowrank_hessian(H, L)
            XL = X @ L
            for w in W:
                s = (w.max() - w.min()) / 3.0
                z = np.round(-w.min() / s)
                for codes in itertools.product(range(4), repeat=n):
                    what = s * (np.asarray(codes, dtype=np.float64) - z)
                    y = X @ (w - what)
                    rho = np.linalg.lstsq(XL, y, rcond=None)[0]
                    best = float(np.sum((y - XL @ rho) ** 2))
                    d = w - what
                    closed = 0.5 * float(d @ HL @ d)
                    assert abs(closed - best) <= 1e-9 * float(np.sum(y ** 2)) + 1e-12
                    R = oracle.lowrank_compensation(w[None, :], what[None, :], K)
                    np.testing.assert_allclose(R[:, 0], rho, rtol=1e-8, atol=1e-10)


def test_lowrank_basis_is_the_truncated_svd():
    X, _, _ = _lora_inputs(32, T=60, n=7, spikes=(9.0, 5.0, 2.5))
    H = 2.0 * X.T @ X
    Vt = np.linalg.svd(X, full_matrices=False)[2]
    for r in (1, 2, 3):
        L = oracle.lowrank_basis(H, r)
        Vr = Vt[:r].T
        np.testing.assert_allclose(L @ L.T, Vr @ Vr.T, atol=1e-10)
        np.testing.assert_allclose(L.T @ L, np.eye(r), atol=1e-12)
        Xp = X - X @ Vr @ Vr.T
        HL, _ = oracle.lowrank_hessian(H, L)
        np.testing.assert_allclose(HL, 2.0 * Xp.T @ Xp, atol=1e-9 * np.max(np.abs(H)))


def test_lowrank_depends_on_the_span_only():
    X, W, rng = _lora_inputs(33, T=50, n=8, m=4)
    H = 2.0 * X.T @ X
    L = np.linalg.qr(rng.standard_normal((8, 3)))[0]
    A = rng.standard_normal((3, 3)) + 3 * np.eye(3)          # any invertible change of basis
    HL1, K1 = oracle.lowrank_hessian(H, L)
    HL2, K2 = oracle.lowrank_hessian(H, L @ A)
    np.testing.assert_allclose(HL1, HL2, atol=1e-10 * np.max(np.abs(H)))
    What = np.round(W * 2) / 2
    C1 = oracle.lowrank_compensation(W, What, K1).T @ L.T
    C2 = oracle.lowrank_compensation(W, What, K2).T @ (L @ A).T
    np.testing.assert_allclose(C1, C2, atol=1e-10)
    # H_L annihilates the span (H_L L = 0) and stays positive semidefinite.
    assert np.max(np.abs(HL1 @ L)) <= 1e-10 * np.max(np.abs(H))
    assert np.min(np.linalg.eigvalsh(HL1)) >= -1e-10 * np.max(np.abs(H))


@pytest.mark.parametrize("levels,group,act", [(4, 0, False), (8, 4, True)])
def test_lora_layer_loss_and_rank_zero(levels, group, act):
    X, W, _ = _lora_inputs(34, T=80, n=12, m=6, spikes=(8.0, 4.0))
    H = 2.0 * X.T @ X
    res = oracle.gptq_lora_layer(W, X=X, rank=2, levels=levels, group_size=group, act_order=act,
                                 damp_rel=0.01, block_size=4)
    D = W - res["What"]
    Dj = D - res["R"].T @ res["L"].T
    direct = float(np.sum((Dj @ X.T) ** 2))
    np.testing.assert_allclose(res["loss_joint"], direct, rtol=1e-9)
    np.testing.assert_allclose(direct, 0.5 * float(np.sum((D @ res["H_aug"]) * D)), rtol=1e-9)
    assert direct <= float(np.sum((D @ X.T) ** 2)) * (1 + 1e-12)     # R* is no worse than R = 0
    r0 = oracle.gptq_lora_layer(W, X=X, rank=0, levels=levels, group_size=group, act_order=act, block_size=4)
    plain = oracle.gptq_layer(W, X=X, levels=levels, group_size=group, act_order=act, block_size=4)
    np.testing.assert_array_equal(r0["codes"], plain["codes"])
    assert r0["R"].shape == (0, W.shape[0])


LOWRANK_MUTATIONS = {
    "M instead of its inverse": ("lowrank_hessian", "K = np.linalg.solve(M, HL.T).T", "K = HL @ M"),
    "downdate sign": ("lowrank_hessian", "return H - K @ HL.T, K", "return H + K @ HL.T, K"),
    "dropped H in H L": ("lowrank_hessian", "HL = H @ L", "HL = L"),
    "compensation sign": ("lowrank_compensation", "D = np.asarray(W, dtype=F64) - np.asarray(What, dtype=F64)",
                          "D = np.asarray(What, dtype=F64) - np.asarray(W, dtype=F64)"),
}


@pytest.mark.parametrize("name", sorted(LOWRANK_MUTATIONS))
def test_lowrank_planted_mistakes_are_caught(name, monkeypatch):
    fn, old, new = LOWRANK_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(getattr(go, fn)))
    assert old in src
    ns = dict(go.__dict__)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(go, fn, ns[fn])
    monkeypatch.setattr(oracle, fn, ns[fn])
    caught = []
    for check in (test_lowrank_hessian_is_the_joint_optimum_over_r, test_lowrank_basis_is_the_truncated_svd,
                  test_lowrank_depends_on_the_span_only):
        try:
            check()
        except AssertionError:
            caught.append(check)
    assert caught, f"mutation '{name}' was not caught by any pin"


# ---------------------------------------------------------------------------
# Planted mistakes in the whole-decoder oracle: each plausible slip in its
# pieces or its wiring must fail at least one decoder pin.
# ---------------------------------------------------------------------------
DECODER_MUTATIONS = {
    "silu with sigmoid(-x)": ("silu", "return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    "silu without x": ("silu", "return x / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(-x))"),
    "swiglu without gate": ("quantize_decoder",
                            'mm = silu(h2 @ res["gate"]["What"].T) * (h2 @ res["up"]["What"].T)',
                            'mm = h2 @ res["up"]["What"].T'),
    "swiglu gate and up swapped": ("quantize_decoder",
                                   'mm = silu(h2 @ res["gate"]["What"].T) * (h2 @ res["up"]["What"].T)',
                                   'mm = silu(h2 @ res["up"]["What"].T) * (h2 @ res["gate"]["What"].T)'),
    "rope sign": ("rope", "x1 * cos - x2 * sin, x1 * sin + x2 * cos", "x1 * cos + x2 * sin, x1 * sin + x2 * cos"),
    "no causal mask": ("attention", "sc = np.where(np.tril(np.ones((seq_len, seq_len), dtype=bool)), sc, -np.inf)",
                       "pass"),
    "rms without root": ("rms_norm", "return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                         "return x / (np.mean(x * x, axis=-1, keepdims=True) + eps)"),
}


@pytest.mark.parametrize("name", sorted(DECODER_MUTATIONS))
def test_decoder_planted_mistakes_are_caught(name, monkeypatch):
    D = oracle.decoder_oracle
    fn, old, new = DECODER_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(getattr(D, fn)))
    assert old in src
    ns = dict(D.__dict__)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    # the module attribute is the entry of the module's globals, which the
    # other decoder functions look the mutant up in
    monkeypatch.setitem(D.__dict__, fn, ns[fn])
    caught = []
    for check in (test_decoder_pieces_closed_forms, test_silu_closed_forms,
                  test_attention_against_explicit_rotations_and_softmax, test_rms_norm_by_hand,
                  lambda: test_decoder_pass_feeds_each_layer_the_quantized_predecessors(4, 32, False)):
        try:
            check()
        except AssertionError:
            caught.append(check)
    assert caught, f"mutation '{name}' was not caught by any pin"
