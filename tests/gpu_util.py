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


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def code_mismatch(gpu_codes, oracle_codes):
    g = np.asarray(gpu_codes).astype(np.int64)
    o = np.asarray(oracle_codes).astype(np.int64)
    return int(np.sum(g != o)), g.size


def log(msg):
    print(msg, flush=True)


# Rounding ties.  Where w/s lies on a rounding boundary either code is a
# correct result, and the sweep then follows another (equally valid) branch
# for the rest of the row.  The fp32 GPU sweep and the fp64 oracle see w/s
# differing by rounding noise, so a row may split at such a point.  A split is
# accepted only when the oracle's w/s at the first differing column is within
# TIE_TOL grid steps of a half-integer; the oracle is then re-run on that row
# with the GPU's code forced there and must agree with the GPU again (repeated
# for further ties in the row).
TIE_TOL = 2e-3
MAX_TIES_PER_ROW = 8


def certify_ties(W64, U64, perm, levels, group, block, codes_gpu, codes_oracle, max_rows=16):
    """Returns (rows_checked, ties) for the rows where codes differ; raises
    AssertionError when a split is not at a near-tie or the forced oracle
    does not converge to the GPU's row."""
    import oracle
    codes_gpu = np.asarray(codes_gpu).astype(np.int64)
    codes_oracle = np.asarray(codes_oracle).astype(np.int64)
    rows = np.nonzero(np.any(codes_gpu != codes_oracle, axis=1))[0]
    assert rows.size <= max_rows, f"{rows.size} rows differ"
    ties = 0
    for r in rows:
        forced = {}
        for _ in range(MAX_TIES_PER_ROW + 1):
            res = oracle.gptq_quantize(W64[r:r + 1], U64, perm, levels, group, block_size=block,
                                       record_inputs=True, forced=forced)
            diff = np.nonzero(res["codes"][0].astype(np.int64) != codes_gpu[r])[0]
            if diff.size == 0:
                break
            j = int(diff[0])
            gi = 0 if group == 0 else j // group
            s = np.float32(res["scales"][0, gi])
            q = np.float32(np.float32(res["qin"][0, j]) / s)
            margin = abs(float(q - np.floor(q)) - 0.5)
            assert margin <= TIE_TOL, f"row {r} column {j}: w/s = {float(q)!r} is {margin:.3g} from a tie"
            forced[(0, j)] = int(codes_gpu[r, j])
            ties += 1
        else:
            raise AssertionError(f"row {r}: more than {MAX_TIES_PER_ROW} ties")
    return int(rows.size), ties
