"""Parity of the asymmetric-calibration path (gptq_asym_target and the
gptaq_quantize_linear sequence, through the C ABI) with the oracle.

Target: both sides take the same float32 H and Hc (the oracle's, rounded),
the GPU its own U from gptq_prepare_hinv; the bar is the float32 rounding
of the three products, |W'_gpu - W'| <= (3n + 16) 2^-24 M with
M = |W| |Hc|^T |U|^T |U| (the oracle's U).  End to end: the GPU forms H and
Hc itself from [Xq | Xf]; codes agree with oracle.gptaq_layer except at
certified rounding ties, relative layer loss within 1e-3.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import certify_ties, dev, host, log, rel_fro, processing_order

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g(gpu_lib):
    import post_weight_quantization_11_amd as g
    return g


def _inputs(T, n, m, seed, noise=0.05):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 51])))
    a = np.exp(rng.normal(0.0, 0.7, size=n))
    Xf = (rng.standard_normal((T, n)) * a).astype(np.float32)
    Xq = (Xf + noise * rng.standard_normal((T, n)) * a).astype(np.float32)
    W = rng.normal(0.0, 0.02, size=(m, n)).astype(np.float32)
    return W, Xq, Xf


@pytest.mark.parametrize("m,n,act", [(96, 200, False), (70, 333, True), (128, 512, True)])
def test_asym_target_parity(g, m, n, act):
    log(f"asym target m={m} n={n} act={act}")
    W, Xq, Xf = _inputs(3 * n, n, m, seed=m + n)
    H = oracle.hessian(Xq.astype(np.float64)).astype(np.float32)
    Hc = (2.0 * (Xq.astype(np.float64).T @ Xf.astype(np.float64))).astype(np.float32)
    U, perm = g.gptq_prepare_hinv(dev(H), 0.01, act)
    Wt = host(g.gptq_asym_target(dev(W), dev(Hc), U, perm if act else None)).astype(np.float64)
    Wo = oracle.asymmetric_target_from_hessians(W, H, Hc, 0.01)
    po = oracle.act_order_perm(H.astype(np.float64)) if act else np.arange(n)
    Hd, _ = oracle.damp_and_permute(H.astype(np.float64), po, 0.01)
    Uo = oracle.inverse_cholesky_upper(Hd)
    Gm = (np.abs(W.astype(np.float64)) @ np.abs(Hc.astype(np.float64)).T)[:, po]
    M = np.empty_like(Gm)
    M[:, po] = (Gm @ np.abs(Uo).T) @ np.abs(Uo)
    err = np.abs(Wt - Wo)
    tol = (3 * n + 16) * 2.0 ** -24 * M
    log(f"  max err/tol = {float(np.max(err / tol)):.3e}, rel_fro = {np.linalg.norm(Wt - Wo) / np.linalg.norm(Wo):.3e}")
    assert np.all(err <= tol)


@pytest.mark.parametrize("levels,group,act,xdt", [(16, 0, False, "f32"), (8, 64, True, "f32"), (4, 32, True, "bf16")])
def test_gptaq_layer_parity(g, levels, group, act, xdt):
    import torch
    from tests.gpu_util import stored_to_dev
    import workloads as wl
    m, n, T = 80, 256, 1500
    log(f"gptaq layer m={m} n={n} tokens={T} levels={levels} group={group} act={act} x={xdt}")
    W, Xq32, Xf32 = _inputs(T, n, m, seed=levels + group)
    Xq, Xf = wl.to_storage(Xq32, xdt), wl.to_storage(Xf32, xdt)
    q = g.gptaq_quantize_linear(dev(W), stored_to_dev(Xq), stored_to_dev(Xf), levels=levels, group_size=group,
                                act_order=act)
    torch.cuda.synchronize()
    ro = oracle.gptaq_layer(W.astype(np.float64), Xq.f32.astype(np.float64), Xf.f32.astype(np.float64),
                            levels=levels, group_size=group, act_order=act)
    if act:
        np.testing.assert_array_equal(host(q["perm"]), ro["perm"])
    cg = processing_order(host(q["codes"]), ro["perm"]).astype(np.int64)
    rows, ties = certify_ties(ro["Wt"], ro["U"], ro["perm"], levels, group, 128, cg, ro["codes"])
    log(f"  rows differing {rows}, ties {ties}")
    assert rows <= max(1, int(1e-4 * cg.size))
    # layer loss on the asymmetric objective: ||Xq Q^T - Xf W^T||^2 with both sides' Q
    Qg = oracle.dequantize(dict(codes=cg.astype(np.float32), scales=host(q["scales"]), zeros=host(q["zeros"]),
                                group_size=group, perm=ro["perm"]))
    Xq64, Xf64 = Xq.f32.astype(np.float64), Xf.f32.astype(np.float64)
    lg = np.sum((Xq64 @ Qg.T - Xf64 @ W.T.astype(np.float64)) ** 2)
    lo = np.sum((Xq64 @ oracle.dequantize(ro).T - Xf64 @ W.T.astype(np.float64)) ** 2)
    log(f"  asymmetric loss gpu {lg:.6e} oracle {lo:.6e}")
    assert abs(lg - lo) <= 1e-3 * lo


@pytest.mark.parametrize("n,tokens,skipped", [(2048, 640, True), (300, 500, False)])
def test_hessian_pair_blocks(g, n, tokens, skipped):
    # gptq_hessian_pair_accumulate writes the Xq^T Xq and Xq^T Xf blocks (and
    # their mirrors) as the full call would; for n a multiple of 2048 the
    # Xf^T Xf block's tiles are skipped, which the untouched sentinel shows.
    import torch
    log(f"hessian pair n={n} tokens={tokens}")
    W, Xq, Xf = _inputs(tokens, n, 8, seed=n + 7)
    Xcat = np.concatenate([Xq, Xf], axis=1)
    H2 = torch.full((2 * n, 2 * n), 12345.0, dtype=torch.float32, device="cuda")
    g.gptq_hessian_pair_accumulate(H2, dev(Xcat), 2.0, reset=True)
    Hg = host(H2).astype(np.float64)
    Ho = oracle.hessian(Xcat.astype(np.float64))
    top = slice(0, n)
    assert rel_fro(Hg[top, top], Ho[top, top]) <= 1e-5
    assert rel_fro(Hg[top, n:], Ho[top, n:]) <= 1e-5
    np.testing.assert_array_equal(Hg[n:, top], Hg[top, n:].T)
    np.testing.assert_array_equal(Hg[top, top], Hg[top, top].T)
    if skipped:
        assert np.all(Hg[n:, n:] == 12345.0)
    else:
        assert rel_fro(Hg[n:, n:], Ho[n:, n:]) <= 1e-5
