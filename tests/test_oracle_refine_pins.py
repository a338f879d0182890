"""Pins of the oracle's fixed-grid refinement (oracle.refine_codes, the
reading of the Daily Papers page's "Bid-Up" step in the GPTQ-intrinsic LoRA
abstract) and of its alternation with the optimal low-rank compensation
(oracle.lora_refine).

None of these re-run the refinement's own arithmetic: each checks it against
enumeration of the grid (a diagonal Hessian makes the problem separable),
brute force over every code vector of a tiny layer, the reconstruction error
computed directly from the calibration inputs X, or a least-squares solve.
"""
import inspect
import itertools
import textwrap

import numpy as np
import pytest

import oracle
from oracle import gptq_oracle as go

F32 = np.float32


def _layer(seed, m, n, tokens, levels, group=0, spikes=()):
    """W, X and a fixed per-row (group=0) or per-group grid from W's ranges."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((tokens, n)) @ (np.eye(n) + 0.4 * rng.standard_normal((n, n)))
    for k, a in enumerate(spikes):
        X += a * np.outer(rng.standard_normal(tokens), rng.standard_normal(n))
    W = rng.standard_normal((m, n)) * 0.5
    gsz = n if group == 0 else group
    G = -(-n // gsz)
    g_idx = (np.arange(n) // gsz).astype(np.int32)
    scales = np.zeros((m, G), F32)
    zeros = np.zeros((m, G), F32)
    for gi in range(G):
        s, z = oracle.grid_params(W[:, gi * gsz:(gi + 1) * gsz], levels - 1)
        scales[:, gi], zeros[:, gi] = s, z
    return W, X, scales, zeros.astype(np.uint8), g_idx


def _what(codes, scales, zeros, g_idx):
    """W^ written out element by element from the grid's definition."""
    m, n = codes.shape
    out = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            s = float(np.float32(scales[i, g_idx[j]]))
            out[i, j] = s * (int(codes[i, j]) - int(zeros[i, g_idx[j]]))
    return out


def _direct_loss_rows(T, What, X):
    """||X (T - W^)_i^T||^2 per row, from X itself (never forms X^T X)."""
    return np.sum(((T - What) @ X.T) ** 2, axis=1)


# ---------------------------------------------------------------------------
# A diagonal Hessian separates the columns: one sweep must land every code on
# the grid value nearest to the target, whatever the starting codes.  The
# nearest value is found by enumerating all levels of the column's grid.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("levels,group", [(16, 0), (4, 4), (3, 0)])
def test_diagonal_hessian_gives_the_nearest_grid_value(levels, group):
    rng = np.random.default_rng(levels + group)
    m, n = 6, 12
    W, _, scales, zeros, g_idx = _layer(3 + levels, m, n, 30, levels, group)
    h = rng.uniform(0.3, 3.0, n)
    H = np.diag(h)
    start = rng.integers(0, levels, (m, n))
    codes, moves = oracle.refine_codes(W, H, start, scales, zeros, g_idx, levels, sweeps=1)
    expect = np.zeros((m, n), np.int64)
    for i in range(m):
        for j in range(n):
            s = float(np.float32(scales[i, g_idx[j]]))
            z = int(zeros[i, g_idx[j]])
            vals = [s * (c - z) for c in range(levels)]
            expect[i, j] = int(np.argmin([(W[i, j] - v) ** 2 for v in vals]))
    np.testing.assert_array_equal(codes, expect)
    assert moves == [int(np.sum(expect != start))]
    # a second sweep finds nothing left to move
    again, moves2 = oracle.refine_codes(W, H, codes, scales, zeros, g_idx, levels, sweeps=1)
    np.testing.assert_array_equal(again, codes)
    assert moves2 == [0]


# ---------------------------------------------------------------------------
# Tiny layer, full Hessian: the error never increases from sweep to sweep,
# and once a sweep makes no move the codes are coordinate-wise optimal:
# changing any one code to any other level does not lower the error
# (checked by brute force over every single change, error from X).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,levels,group", [(1, 3, 0), (2, 4, 2), (3, 16, 0), (4, 4, 0)])
def test_monotone_and_coordinatewise_optimal(seed, levels, group):
    m, n = 5, 6
    W, X, scales, zeros, g_idx = _layer(seed, m, n, 14, levels, group)
    H = 2.0 * X.T @ X
    rng = np.random.default_rng(seed + 100)
    codes = rng.integers(0, levels, (m, n))
    prev = _direct_loss_rows(W, _what(codes, scales, zeros, g_idx), X)
    for _ in range(60):
        codes, moves = oracle.refine_codes(W, H, codes, scales, zeros, g_idx, levels, sweeps=1)
        cur = _direct_loss_rows(W, _what(codes, scales, zeros, g_idx), X)
        assert np.all(cur <= prev * (1 + 1e-12))
        prev = cur
        if moves == [0]:
            break
    assert moves == [0]
    for i, j in itertools.product(range(m), range(n)):
        for c in range(levels):
            alt = codes.copy()
            alt[i, j] = c
            li = _direct_loss_rows(W[i:i + 1], _what(alt[i:i + 1], scales[i:i + 1], zeros[i:i + 1], g_idx), X)[0]
            assert li >= prev[i] * (1 - 1e-12), (i, j, c)


# ---------------------------------------------------------------------------
# Started at the global optimum (every code vector of the row enumerated),
# the refinement moves nothing; started anywhere, it never ends above where
# it began and never below that optimum.
# ---------------------------------------------------------------------------
def test_global_optimum_is_a_fixed_point():
    levels, m, n = 3, 3, 5
    W, X, scales, zeros, g_idx = _layer(9, m, n, 12, levels)
    H = 2.0 * X.T @ X
    best = np.zeros((m, n), np.int64)
    best_loss = np.zeros(m)
    for i in range(m):
        cands = np.array(list(itertools.product(range(levels), repeat=n)))
        losses = _direct_loss_rows(np.repeat(W[i:i + 1], len(cands), 0),
                                   _what(cands, np.repeat(scales[i:i + 1], len(cands), 0),
                                         np.repeat(zeros[i:i + 1], len(cands), 0), g_idx), X)
        best[i] = cands[int(np.argmin(losses))]
        best_loss[i] = losses.min()
    codes, moves = oracle.refine_codes(W, H, best, scales, zeros, g_idx, levels, sweeps=2)
    np.testing.assert_array_equal(codes, best)
    assert moves == [0, 0]
    start = np.random.default_rng(0).integers(0, levels, (m, n))
    out, _ = oracle.refine_codes(W, H, start, scales, zeros, g_idx, levels, sweeps=5)
    lo = _direct_loss_rows(W, _what(out, scales, zeros, g_idx), X)
    assert np.all(lo >= best_loss * (1 - 1e-12))
    assert np.all(lo <= _direct_loss_rows(W, _what(start, scales, zeros, g_idx), X) * (1 + 1e-12))


# ---------------------------------------------------------------------------
# Edges: a column whose input is always zero (H_jj = 0) keeps its codes;
# zero sweeps change nothing.
# ---------------------------------------------------------------------------
def test_dead_column_and_zero_sweeps():
    levels, m, n = 4, 4, 6
    W, X, scales, zeros, g_idx = _layer(5, m, n, 20, levels)
    X[:, 2] = 0.0
    H = 2.0 * X.T @ X
    start = np.random.default_rng(1).integers(0, levels, (m, n))
    codes, _ = oracle.refine_codes(W, H, start, scales, zeros, g_idx, levels, sweeps=3)
    np.testing.assert_array_equal(codes[:, 2], start[:, 2])
    assert np.any(codes != start)
    same, moves = oracle.refine_codes(W, H, start, scales, zeros, g_idx, levels, sweeps=0)
    np.testing.assert_array_equal(same, start)
    assert moves == []


# ---------------------------------------------------------------------------
# Alternation with the compensation, both forms: the joint error
# ||X (W - W^ - R^T L^T)^T||^2 (computed from X) never increases from round
# to round and the final R is the least-squares optimum for the final codes
# (a least-squares solve on X L, which does not use the compensation's
# formula).  Literal form: the refinement with R held fixed lowers exactly
# that error with R fixed.  Joint form: once a round changes nothing, no
# single change of a code lowers min over R of the joint error (brute force
# over every single change, each with its own least-squares R).
# ---------------------------------------------------------------------------
def _min_over_r(W, What, X, L):
    XL = X @ L
    D = W - What
    R = np.linalg.lstsq(XL, X @ D.T, rcond=None)[0]
    return np.sum(((D - R.T @ L.T) @ X.T) ** 2, axis=1), R


@pytest.mark.parametrize("joint", [False, True])
@pytest.mark.parametrize("rank,levels,group", [(1, 3, 0), (2, 4, 2), (3, 16, 0)])
def test_alternation_with_the_compensation(rank, levels, group, joint):
    m, n = 4, 6
    W, X, scales, zeros, g_idx = _layer(20 + rank, m, n, 40, levels, group, spikes=(5.0, 3.0, 2.0)[:rank])
    H = 2.0 * X.T @ X
    L = oracle.lowrank_basis(H, rank)
    HL, _ = oracle.lowrank_hessian(H, L)
    res = oracle.gptq_layer(W, H=HL, levels=levels, group_size=group if group else 0, damp_rel=0.01)
    sc, ze, gi = res["scales"], res["zeros"].astype(np.uint8), res["g_idx"]
    codes0 = res["codes_orig"]
    codes, R, losses = oracle.lora_refine(W, H, L, codes0, sc, ze, gi, levels, rounds=3, sweeps=1, joint=joint)
    What = _what(codes, sc, ze, gi)
    rows, Rls = _min_over_r(W, What, X, L)
    np.testing.assert_allclose(R, Rls, rtol=1e-8, atol=1e-10)
    direct = float(np.sum(((W - What - R.T @ L.T) @ X.T) ** 2))
    np.testing.assert_allclose(losses[-1], direct, rtol=1e-9)
    np.testing.assert_allclose(direct, rows.sum(), rtol=1e-9)
    assert all(b <= a * (1 + 1e-12) for a, b in zip(losses, losses[1:]))
    if np.any(codes != codes0):
        assert losses[-1] < losses[0]
    # from arbitrary codes on the same grid the alternation must make progress
    start = np.random.default_rng(rank).integers(0, levels, codes0.shape)
    _, _, lr = oracle.lora_refine(W, H, L, start, sc, ze, gi, levels, rounds=2, sweeps=1, joint=joint)
    assert lr[0] > lr[1] >= lr[2] * (1 - 1e-12)
    if not joint:
        # the refinement step itself, R held at its value before the last round
        c_prev, R_prev, _ = oracle.lora_refine(W, H, L, codes0, sc, ze, gi, levels, rounds=2, sweeps=1, joint=False)
        c_step, _ = oracle.refine_codes(W, H, c_prev, sc, ze, gi, levels, sweeps=1, L=L, R=R_prev)
        T = W - R_prev.T @ L.T
        before = np.sum(((T - _what(c_prev, sc, ze, gi)) @ X.T) ** 2)
        after = np.sum(((T - _what(c_step, sc, ze, gi)) @ X.T) ** 2)
        assert after <= before * (1 + 1e-12)
        np.testing.assert_array_equal(c_step, codes)
        return
    # joint form, run to its fixed point from the arbitrary start
    c = start
    for _ in range(40):
        c_new, _, _ = oracle.lora_refine(W, H, L, c, sc, ze, gi, levels, rounds=1, sweeps=1, joint=True)
        if np.array_equal(c_new, c):
            break
        c = c_new
    assert np.array_equal(c_new, c)
    best, _ = _min_over_r(W, _what(c, sc, ze, gi), X, L)
    for i, j in itertools.product(range(m), range(n)):
        for cc in range(levels):
            alt = c.copy()
            alt[i, j] = cc
            li, _ = _min_over_r(W, _what(alt, sc, ze, gi), X, L)
            assert li[i] >= best[i] * (1 - 1e-9), (i, j, cc)


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the refinement must fail a pin.
# ---------------------------------------------------------------------------
REFINE_MUTATIONS = {
    "gradient update sign": ("refine_codes", "g -= delta * H[:, j]", "g += delta * H[:, j]"),
    "stale gradient": ("refine_codes", "g -= delta * H[:, j]", "pass"),
    "step without H_jj": ("refine_codes", "v = what[j] + g[j] / hjj", "v = what[j] + g[j]"),
    "zero point dropped": ("refine_codes", "np.rint(v / S[i, j]) + Z[i, j]", "np.rint(v / S[i, j])"),
    "gain test inverted": ("refine_codes", "if not gain > 0:", "if not gain < 0:"),
    "correction ignored": ("refine_codes", "T = T - np.asarray(R, dtype=F64).T @ np.asarray(L, dtype=F64).T",
                           "pass"),
}


@pytest.mark.parametrize("name", sorted(REFINE_MUTATIONS))
def test_refine_planted_mistakes_are_caught(name, monkeypatch):
    fn, old, new = REFINE_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(getattr(go, fn)))
    assert old in src
    ns = dict(go.__dict__)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(go, fn, ns[fn])
    monkeypatch.setattr(oracle, fn, ns[fn])
    caught = []
    for check in (lambda: test_diagonal_hessian_gives_the_nearest_grid_value(16, 0),
                  lambda: test_monotone_and_coordinatewise_optimal(1, 3, 0),
                  lambda: test_monotone_and_coordinatewise_optimal(3, 16, 0),
                  lambda: test_alternation_with_the_compensation(2, 4, 2, False),
                  lambda: test_alternation_with_the_compensation(2, 4, 2, True)):
        try:
            check()
        except AssertionError:
            caught.append(check)
    assert caught, f"mutation '{name}' was not caught by any pin"
