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


def test_certify_accepts_a_branch_at_admitted_ties(monkeypatch):
    W, U, _, res = _case(group=8)
    res = oracle.gptq_quantize(W, U, None, 16, 8, block_size=16, record_inputs=True)
    forced = {(0, 3): (int(res["codes"][0, 3]) + 1) % 16, (4, 17): (int(res["codes"][4, 17]) + 3) % 16}
    branch = oracle.gptq_quantize(W, U, None, 16, 8, block_size=16, forced=forced)
    monkeypatch.setattr(gu, "TIE_TOL", 0.5)   # every decision counts as a tie here
    rows, ties = gu.certify_ties(W, U, None, 16, 8, 16, branch["codes"], res["codes"])
    assert rows == 2 and ties == 2
    # identical codes: nothing to certify
    assert gu.certify_ties(W, U, None, 16, 8, 16, res["codes"], res["codes"]) == (0, 0)
