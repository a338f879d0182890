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
