"""CPU checks of the oracle's forced-decision option and of the rounding-tie
certification that the GPU parity tests apply when the fp32 sweep takes the
other branch at a tie (either code is correct there)."""
import numpy as np
import pytest

import oracle
import tests.gpu_util as gu


def _case(m=6, n=40, seed=3, levels=16, group=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((3 * n, n)) @ (np.eye(n) + rng.standard_normal((n, n)) / np.sqrt(n))
    H = oracle.hessian(X)
    Hd, _ = oracle.damp_and_permute(H, None, 0.01)
    U = oracle.inverse_cholesky_upper(Hd)
    W = rng.standard_normal((m, n)) * 0.02
    res = oracle.gptq_quantize(W, U, None, levels, group, block_size=16, record_inputs=True)
    return W, U, Hd, res


def test_forced_branch_is_a_consistent_gptq_trajectory():
    W, U, Hd, res = _case()
    r, j = 2, 5
    c = int(res["codes"][r, j])
    alt = c + 1 if c < 15 else c - 1
    f = oracle.gptq_quantize(W, U, None, 16, 0, block_size=16, forced={(r, j): alt})
    assert f["codes"][r, j] == alt
    # columns before j and the other rows are untouched
    np.testing.assert_array_equal(f["codes"][r, :j], res["codes"][r, :j])
    others = np.arange(W.shape[0]) != r
    np.testing.assert_array_equal(f["codes"][others], res["codes"][others])
    # the loss identity still holds on the forced branch (errors propagated)
    What = oracle.dequantize(f)
    obs = oracle.obs_loss(W, What, Hd, np.arange(W.shape[1]))
    np.testing.assert_allclose(obs, f["row_loss"], rtol=1e-10)
    # forcing the code the oracle chose changes nothing
    same = oracle.gptq_quantize(W, U, None, 16, 0, block_size=16, forced={(r, j): c})
    np.testing.assert_array_equal(same["codes"], res["codes"])


def test_certify_rejects_a_flip_away_from_a_tie():
    W, U, _, res = _case()
    r = 1
    q = np.float32(np.float32(res["qin"][r]) / np.float32(res["scales"][r, 0]))
    margins = np.abs((q - np.floor(q)) - 0.5)
    j = int(np.argmax(margins))          # the decision farthest from a tie
    assert margins[j] > 0.1
    c = int(res["codes"][r, j])
    alt = c + 1 if c < 15 else c - 1
    branch = oracle.gptq_quantize(W, U, None, 16, 0, block_size=16, forced={(r, j): alt})
    with pytest.raises(AssertionError, match="from a tie"):
        gu.certify_ties(W, U, None, 16, 0, 16, branch["codes"], res["codes"])


def _adjacent(res, r, j):
    """The other code adjacent to the oracle's w/s at (r, j)."""
    g = res["group_size"]
    gi = 0 if g == 0 else j // g
    s, z = np.float32(res["scales"][r, gi]), int(res["zeros"][r, gi])
    q = np.float32(np.float32(res["qin"][r, j]) / s)
    lo, hi = int(np.floor(q)) + z, int(np.floor(q)) + 1 + z
    c = int(res["codes"][r, j])
    return hi if c == lo else lo


def test_certify_rejects_a_code_not_adjacent_to_the_tie(monkeypatch):
    W, U, _, res = _case(group=8)
    res = oracle.gptq_quantize(W, U, None, 16, 8, block_size=16, record_inputs=True)
    c = int(res["codes"][2, 9])
    branch = oracle.gptq_quantize(W, U, None, 16, 8, block_size=16, forced={(2, 9): (c + 3) % 16})
    monkeypatch.setattr(gu, "K_SIGMA", 1e12)
    with pytest.raises(AssertionError, match="not adjacent"):
        gu.certify_ties(W, U, None, 16, 8, 16, branch["codes"], res["codes"])


def _fp32_sweep(W, U, levels, group, scales_out=None):
    """The unblocked sweep with every operation rounded to float32 (values
    recorded when quantized): a float32 computation of the same decisions.
    With scales_out (a list), each group's scales are appended to it."""
    f = np.float32
    W = np.asarray(W, dtype=f)
    U = np.asarray(U, dtype=f)
    m, n = W.shape
    maxq = levels - 1
    V = W.copy()
    qin = np.zeros((m, n), dtype=f)
    codes = np.zeros((m, n), dtype=f)
    if group == 0:
        s, z = oracle.grid_params(V, maxq)
        if scales_out is not None:
            scales_out.append(s)
    for j in range(n):
        if group and j % group == 0:
            s, z = oracle.grid_params(V[:, j:j + group], maxq)
            if scales_out is not None:
                scales_out.append(s)
        v = V[:, j].copy()
        qin[:, j] = v
        c = oracle.quantize_values(v, s, z, maxq)
        what = (s * (c - z)).astype(f)
        e = ((v - what).astype(f) * f(f(1) / U[j, j])).astype(f)
        codes[:, j] = c
        V[:, j + 1:] = (V[:, j + 1:] - (e[:, None] * U[j, j + 1:][None, :]).astype(f)).astype(f)
    return codes, qin


@pytest.mark.parametrize("group", [0, 16, 8, 2])
def test_fp32_sweep_deviation_within_the_derived_sigma(group):
    # The tolerance model must not be optimistic: a float32 sweep's values
    # deviate from the float64 oracle's by less than K_SIGMA sigma_j at every
    # column before the first code difference of a row (and by far less in rms).
    rng = np.random.default_rng(31)
    n, m = 384, 48
    X = rng.standard_normal((4 * n, n)) @ (np.eye(n) + rng.standard_normal((n, n)) / np.sqrt(n))
    X *= np.exp(rng.normal(0, 1, n))
    H = oracle.hessian(X)
    Hd, _ = oracle.damp_and_permute(H, None, 0.01)
    U = oracle.inverse_cholesky_upper(Hd).astype(np.float32).astype(np.float64)
    W = (rng.standard_normal((m, n)) * 0.02).astype(np.float32).astype(np.float64)
    res = oracle.gptq_quantize(W, U, None, 16, group, block_size=1, record_inputs=True)
    sigma = gu.sweep_sigma(W, U, None, res)
    c32, q32 = _fp32_sweep(W, U, 16, group)
    ratios = []
    for r in range(m):
        d = np.nonzero(c32[r] != res["codes"][r])[0]
        upto = d[0] if d.size else n
        dev = np.abs(q32[r, :upto].astype(np.float64) - res["qin"][r, :upto])
        assert np.all(dev <= gu.K_SIGMA * sigma[r, :upto] + 1e-30), r
        ratios.append(dev / np.maximum(sigma[r, :upto], 1e-300))
    ratios = np.concatenate(ratios)
    assert np.sqrt(np.mean(ratios ** 2)) < 1.0


@pytest.mark.parametrize("group,levels", [(1, 4), (2, 16), (4, 8), (8, 3)])
def test_small_group_scale_bound_holds_for_a_float32_sweep(group, levels):
    # Scales of groups of 1-8 columns come from one or a few error-updated
    # values; a float32 sweep's scales stay within small_group_scale_bound
    # of the float64 oracle's on every row whose codes agree, and the bound
    # is tight enough to mean something (well under the values' magnitude).
    rng = np.random.default_rng(41 + group)
    n, m = 256, 40
    X = rng.standard_normal((4 * n, n)) @ (np.eye(n) + rng.standard_normal((n, n)) / np.sqrt(n))
    X *= np.exp(rng.normal(0, 1, n))
    Hd, _ = oracle.damp_and_permute(oracle.hessian(X), None, 0.01)
    U = oracle.inverse_cholesky_upper(Hd).astype(np.float32).astype(np.float64)
    W = (rng.standard_normal((m, n)) * 0.02).astype(np.float32).astype(np.float64)
    rec = oracle.gptq_quantize(W, U, None, levels, group, block_size=1, record_inputs=True)
    sc = []
    c32, _ = _fp32_sweep(W, U, levels, group, scales_out=sc)
    s32 = np.stack(sc, axis=1).astype(np.float64)
    ok = np.all(c32 == rec["codes"], axis=1)
    assert ok.sum() >= m // 2
    tol = gu.small_group_scale_bound(W, U, None, rec)
    so = np.asarray(rec["scales"], dtype=np.float64)
    assert np.all(np.abs(s32[ok] - so[ok]) <= tol[ok])
    assert np.median(tol[ok] / so[ok]) < 1e-3


def test_certify_accepts_a_branch_at_admitted_ties(monkeypatch):
    W, U, _, res = _case(group=8)
    res = oracle.gptq_quantize(W, U, None, 16, 8, block_size=16, record_inputs=True)
    forced = {(0, 3): _adjacent(res, 0, 3), (4, 17): _adjacent(res, 4, 17)}
    branch = oracle.gptq_quantize(W, U, None, 16, 8, block_size=16, forced=forced)
    monkeypatch.setattr(gu, "K_SIGMA", 1e12)   # every decision counts as a tie here
    branches = {}
    rows, ties = gu.certify_ties(W, U, None, 16, 8, 16, branch["codes"], res["codes"], branches=branches)
    assert rows == 2 and ties == 2
    # the oracle on the GPU's branches reproduces the branch exactly (losses included)
    on = gu.on_gpu_branches(res, branches)
    np.testing.assert_array_equal(on["codes"], branch["codes"])
    np.testing.assert_array_equal(on["scales"], branch["scales"])
    np.testing.assert_allclose(on["row_loss"], branch["row_loss"], rtol=1e-12)
    assert sorted(branches) == [0, 4]
    # identical codes: nothing to certify
    assert gu.certify_ties(W, U, None, 16, 8, 16, res["codes"], res["codes"]) == (0, 0)
