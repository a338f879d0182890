"""Helpers for GPU tests: host <-> device transfer of workload arrays and the
comparison metrics of the parity bars."""
import numpy as np


def dev(arr, dtype="f32"):
    """numpy -> contiguous cuda tensor.  dtype 'bf16' expects uint16 bit patterns."""
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "f16":
        return torch.from_numpy(a.astype(np.float16)).cuda()
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32)).cuda()
    if dtype == "i32":
        return torch.from_numpy(a.astype(np.int32)).cuda()
    if dtype == "u8":
        return torch.from_numpy(a.astype(np.uint8)).cuda()
    raise ValueError(dtype)


def stored_to_dev(st):
    return dev(st.raw, st.dtype)


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def processing_order(codes, perm):
    """Codes in original column order (as gptq_quantize_layer returns them)
    re-indexed by processing position: column j is original column perm[j]."""
    codes = np.asarray(codes)
    return codes if perm is None else codes[:, np.asarray(perm, dtype=np.int64)]


def expected_wq(codes_orig, scales, zeros, g_idx, dtype):
    """fl_w(fl32(s (c - z))) of each original column, in storage bit patterns
    (bf16 as uint16), from a result's own codes, scales, zeros and g_idx."""
    import workloads as wl
    gi = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scales, dtype=np.float32)[:, gi]
    cz = (np.asarray(codes_orig, dtype=np.float32) - np.asarray(zeros, dtype=np.float32)[:, gi])
    v = (s * cz).astype(np.float32)
    return wl.to_storage(v, dtype).raw


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def code_mismatch(gpu_codes, oracle_codes):
    g = np.asarray(gpu_codes).astype(np.int64)
    o = np.asarray(oracle_codes).astype(np.int64)
    return int(np.sum(g != o)), g.size


def log(msg):
    """Prints msg and keeps it for the run's terminal summary."""
    print(msg, flush=True)
    try:
        from tests.conftest import REPORT_LINES
        REPORT_LINES.append(str(msg))
    except ImportError:  # pragma: no cover
        pass


# Rounding ties.  Where w/s lies on a rounding boundary either code is a
# correct result, and the sweep then follows another (equally valid) branch
# for the rest of the row.  The fp32 GPU sweep and the fp64 oracle see w/s
# differing by rounding noise, so a row may split at such a point.  A split is
# accepted only when (a) the GPU's code is one of the two codes adjacent to
# the oracle's w/s, (b) the oracle's w/s at the first differing column lies
# within the tolerance tau_j of a half-integer, where tau_j is derived below
# from the fp32 sweep's rounding error, and (c) the oracle, re-run on that row
# with the GPU's code forced there, agrees with the GPU again (repeated for
# further ties in the row).
#
# tau_j (grid steps) = K_SIGMA * sigma_j / s + 2 u |q_j| + u |w_j| / s, where
# u = 2^-24 and sigma_j bounds the standard deviation of the GPU's value w_j
# at the moment column j is quantized, under the usual model of rounding
# errors as independent, uniform in [-u, u] relative to the rounded value:
#   * w_j = W_j - sum_{k<j} e_k U_kj is accumulated in float32 with at most
#     j + 2 roundings, each of a partial sum no larger than
#     A_j = |W_j| + sum_{k<j} |e_k U_kj|:   variance <= (j + 2) (u^2/3) A_j^2;
#   * e_k = (w_k - s (c_k - z)) * fl(1/U_kk) adds four roundings of values no
#     larger than (|w_k| + |w^_k|) / U_kk, and carries dw_k / U_kk;
#   * so Var(dw_j) = r_j + sum_{k<j} (U_kj / U_kk)^2 Var(dw_k), with
#     r_j = (j + 2)(u^2/3) A_j^2 + sum_{k<j} U_kj^2 4 (u^2/3) ((|w_k| + |w^_k|)/U_kk)^2,
#     a lower-triangular system solved for all j at once.
# The 2 u |q| and u |w| / s terms are the float32 roundings of w and of the
# quotient on either side.  tests/test_tie_certification.py checks that the
# model is not optimistic: an fp32 sweep's measured deviations from the
# float64 oracle stay below K_SIGMA sigma_j.
U_F32 = 2.0 ** -24
K_SIGMA = 6.0
MAX_TIES_PER_ROW = 8


def sweep_sigma(W64, U64, perm, res):
    """sigma_j (absolute) of every row of ``res`` (an oracle result recorded
    with record_inputs=True for the rows W64) in processing order."""
    from scipy.linalg import solve_triangular
    W64 = np.asarray(W64, dtype=np.float64)
    U = np.asarray(U64, dtype=np.float64)
    n = U.shape[0]
    perm = np.arange(n) if perm is None else np.asarray(perm)
    Wp = np.abs(W64[:, perm])
    E = np.asarray(res["E"], dtype=np.float64)
    d = np.diag(U)
    Uu = np.triu(U, 1)                                  # U_kj, k < j
    A = Wp + np.abs(E) @ np.abs(Uu)                     # A_j per row
    j2 = np.arange(n, dtype=np.float64) + 2.0
    g = np.asarray(res["group_size"])
    gi = np.zeros(n, dtype=np.int64) if int(g) == 0 else np.arange(n) // int(g)
    s = np.asarray(res["scales"], dtype=np.float64)[:, gi]
    z = np.asarray(res["zeros"], dtype=np.float64)[:, gi]
    what = s * (np.asarray(res["codes"], dtype=np.float64) - z)
    qin = np.abs(np.asarray(res["qin"], dtype=np.float64))
    ek = 4.0 * (U_F32 ** 2 / 3.0) * ((qin + np.abs(what)) / d[None, :]) ** 2
    r = j2[None, :] * (U_F32 ** 2 / 3.0) * A ** 2 + ek @ (Uu ** 2)
    M2 = (Uu / d[:, None]) ** 2                         # (U_kj / U_kk)^2, k < j
    var = solve_triangular(np.eye(n) - M2.T, r.T, lower=True)
    return np.sqrt(np.maximum(var.T, 0.0))


def small_group_scale_bound(W64, U64, perm, rec):
    """Allowed absolute scale error per (row, group) for groups of 1-8
    columns, from an oracle result recorded with record_inputs=True: such a
    group's range comes from one or a few error-updated values, each off by
    at most K_SIGMA sigma_k + u |w_k| in a float32 sweep, so the scale
    (range / maxq) is off by at most twice the largest of those over maxq,
    plus three float32 roundings of its own; never below the 1e-5 relative
    bar."""
    g = int(rec["group_size"])
    so = np.asarray(rec["scales"], dtype=np.float64)
    ew = K_SIGMA * sweep_sigma(W64, U64, perm, rec) + U_F32 * np.abs(np.asarray(rec["qin"], dtype=np.float64))
    ewg = np.zeros_like(so)
    for gi in range(so.shape[1]):
        ewg[:, gi] = np.max(ew[:, gi * g:(gi + 1) * g], axis=1)
    return np.maximum(1e-5 * so, 2.0 * ewg / (int(rec["levels"]) - 1) + 3 * U_F32 * so)


def certify_ties(W64, U64, perm, levels, group, block, codes_gpu, codes_oracle, max_rows=16, branches=None):
    """Returns (rows_checked, ties) for the rows where codes differ; raises
    AssertionError when a split is not at a near-tie, when the GPU's code is
    not adjacent to the tie, or when the forced oracle does not converge to
    the GPU's row.  With a dict `branches`, branches[r] receives the oracle's
    result for row r on the GPU's branch (its codes equal the GPU's row)."""
    import oracle
    codes_gpu = np.asarray(codes_gpu).astype(np.int64)
    codes_oracle = np.asarray(codes_oracle).astype(np.int64)
    rows = np.nonzero(np.any(codes_gpu != codes_oracle, axis=1))[0]
    assert rows.size <= max_rows, f"{rows.size} rows differ"
    maxq = levels - 1
    ties = 0
    if rows.size:
        first = oracle.gptq_quantize(W64[rows], U64, perm, levels, group, block_size=block, record_inputs=True)
        sigmas = sweep_sigma(W64[rows], U64, perm, first)
    for ri, r in enumerate(rows):
        forced = {}
        sigma = sigmas[ri]
        for _ in range(MAX_TIES_PER_ROW + 1):
            res = oracle.gptq_quantize(W64[r:r + 1], U64, perm, levels, group, block_size=block,
                                       record_inputs=True, forced=forced)
            diff = np.nonzero(res["codes"][0].astype(np.int64) != codes_gpu[r])[0]
            if diff.size == 0:
                if branches is not None:
                    branches[int(r)] = res
                break
            j = int(diff[0])
            gi = 0 if group == 0 else j // group
            s = np.float32(res["scales"][0, gi])
            z = int(res["zeros"][0, gi])
            w = float(res["qin"][0, j])
            q = np.float32(np.float32(w) / s)
            tol = K_SIGMA * sigma[j] / float(s) + 2 * U_F32 * abs(float(q)) + U_F32 * abs(w) / float(s)
            margin = abs(float(q - np.floor(q)) - 0.5)
            assert margin <= tol, (f"row {r} column {j}: w/s = {float(q)!r} is {margin:.3g} from a tie "
                                   f"(tolerance {tol:.3g})")
            adjacent = {min(max(int(np.floor(q)) + z, 0), maxq), min(max(int(np.floor(q)) + 1 + z, 0), maxq)}
            assert int(codes_gpu[r, j]) in adjacent, (f"row {r} column {j}: GPU code {int(codes_gpu[r, j])} is "
                                                      f"not adjacent to the tie at w/s = {float(q)!r}")
            forced[(0, j)] = int(codes_gpu[r, j])
            ties += 1
        else:
            raise AssertionError(f"row {r}: more than {MAX_TIES_PER_ROW} ties")
    return int(rows.size), ties


def on_gpu_branches(res, branches):
    """The oracle result `res` (rows x n, processing order) with each row r in
    `branches` replaced by the oracle's result on the GPU's branch."""
    out = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in res.items()}
    for r, b in branches.items():
        for key in ("codes", "scales", "zeros", "E", "row_loss"):
            out[key][r] = b[key][0]
    return out
