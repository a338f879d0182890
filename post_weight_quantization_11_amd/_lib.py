"""Thin ctypes binding of libgptq.so (argument marshalling only).

Every computation runs in the HIP kernels of libgptq.so; this module only
turns torch tensors into device pointers, allocates outputs and workspaces
with torch, passes the current HIP stream, and maps status codes to
exceptions.  The functions carry the C entry points' names.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptq.so")

GPTQ_OK = 0
GPTQ_ERR_INVALID_ARG = 1
GPTQ_ERR_UNSUPPORTED = 2
GPTQ_ERR_WORKSPACE = 3
GPTQ_ERR_NOT_PD = 4
GPTQ_ERR_HIP = 5

GPTQ_F32, GPTQ_F16, GPTQ_BF16 = 0, 1, 2

EXPORTS = (
    "gptq_status_string",
    "gptq_hessian_ws_bytes",
    "gptq_hessian_accumulate",
    "gptq_hessian_accumulate_noalloc",
    "gptq_hessian_pair_ws_bytes",
    "gptq_hessian_pair_accumulate",
    "gptq_prepare_ws_bytes",
    "gptq_prepare_hinv",
    "gptq_quantize_ws_bytes",
    "gptq_quantize_layer",
    "gptq_pack",
    "gptq_dequant_gemv",
    "gptq_dequant_gemm",
    "gptq_asym_target_ws_bytes",
    "gptq_asym_target",
    "gptq_lowrank_ws_bytes",
    "gptq_lowrank_basis",
    "gptq_lowrank_hessian",
    "gptq_lowrank_compensation",
    "gptq_refine_ws_bytes",
    "gptq_refine_codes",
)

GEMV_MAX_BATCH = 8   # X rows per pass of the VALU product kernel
LOWRANK_MAX_RANK = 64

_lib = None


class GptqError(RuntimeError):
    def __init__(self, status: int, where: str, info: int = 0):
        self.status = status
        self.info = info
        name = _lib.gptq_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {name}" + (f" (info={info})" if info else ""))


def load(path: str = LIB_PATH):
    """Load libgptq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libgptq.so not built at {path}; run "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    i64, vp, sz, i32p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32)
    C = ctypes.c_int
    lib.gptq_status_string.restype = ctypes.c_char_p
    lib.gptq_status_string.argtypes = [C]
    lib.gptq_hessian_ws_bytes.restype = sz
    lib.gptq_hessian_ws_bytes.argtypes = [i64, i64, C]
    lib.gptq_hessian_accumulate.restype = C
    lib.gptq_hessian_accumulate.argtypes = [vp, i64, vp, C, i64, i64, ctypes.c_float, C, vp, sz, vp]
    lib.gptq_hessian_accumulate_noalloc.restype = C
    lib.gptq_hessian_accumulate_noalloc.argtypes = [vp, i64, vp, C, i64, i64, ctypes.c_float, C, vp]
    lib.gptq_hessian_pair_ws_bytes.restype = sz
    lib.gptq_hessian_pair_ws_bytes.argtypes = [i64, i64, C]
    lib.gptq_hessian_pair_accumulate.restype = C
    lib.gptq_hessian_pair_accumulate.argtypes = [vp, i64, vp, C, i64, i64, ctypes.c_float, C, vp, sz, vp]
    lib.gptq_prepare_ws_bytes.restype = sz
    lib.gptq_prepare_ws_bytes.argtypes = [i64]
    lib.gptq_prepare_hinv.restype = C
    lib.gptq_prepare_hinv.argtypes = [vp, i64, ctypes.c_float, C, vp, vp, i32p, vp, sz, vp]
    lib.gptq_quantize_ws_bytes.restype = sz
    lib.gptq_quantize_ws_bytes.argtypes = [i64, i64, C]
    lib.gptq_quantize_layer.restype = C
    lib.gptq_quantize_layer.argtypes = [vp, C, i64, i64, i64, vp, vp, C, C, C, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gptq_pack.restype = C
    lib.gptq_pack.argtypes = [vp, i64, i64, C, vp, i64, vp]
    lib.gptq_dequant_gemv.restype = C
    lib.gptq_dequant_gemv.argtypes = [vp, i64, i64, i64, C, vp, vp, i64, C, vp, vp, i64, i64, vp, i64, vp]
    lib.gptq_asym_target_ws_bytes.restype = sz
    lib.gptq_asym_target_ws_bytes.argtypes = [i64, i64]
    lib.gptq_asym_target.restype = C
    lib.gptq_asym_target.argtypes = [vp, C, i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, sz, vp]
    lib.gptq_dequant_gemm.restype = C
    lib.gptq_dequant_gemm.argtypes = [vp, i64, i64, i64, C, vp, vp, i64, C, vp, vp, i64, i64, vp, i64, vp]
    lib.gptq_lowrank_ws_bytes.restype = sz
    lib.gptq_lowrank_ws_bytes.argtypes = [i64, i64, i64]
    lib.gptq_lowrank_basis.restype = C
    lib.gptq_lowrank_basis.argtypes = [vp, i64, i64, i64, vp, C, vp, vp, sz, vp]
    lib.gptq_lowrank_hessian.restype = C
    lib.gptq_lowrank_hessian.argtypes = [vp, i64, i64, vp, i64, vp, i64, vp, vp, sz, vp]
    lib.gptq_lowrank_compensation.restype = C
    lib.gptq_lowrank_compensation.argtypes = [vp, C, i64, i64, i64, vp, vp, vp, C, vp, vp, i64, vp, i64, vp, sz,
                                              vp]
    lib.gptq_refine_ws_bytes.restype = sz
    lib.gptq_refine_ws_bytes.argtypes = [i64, i64]
    lib.gptq_refine_codes.restype = C
    lib.gptq_refine_codes.argtypes = [vp, C, i64, i64, i64, vp, i64, vp, vp, i64, i64, vp, vp, C, vp, C, C, vp, vp,
                                      vp, sz, vp]
    _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    return {torch.float32: GPTQ_F32, torch.float16: GPTQ_F16, torch.bfloat16: GPTQ_BF16}[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, where: str, info: int = 0):
    if rc != GPTQ_OK:
        raise GptqError(rc, where, info)


def _workspace(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def _device_check(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def _rows_check(t):
    """Row-major with unit column stride (any leading dimension)."""
    if not t.is_cuda or t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D device tensor with unit column stride")


def gptq_hessian_accumulate(H, X, alpha: float = 2.0, reset: bool = False, ws=None, stream=None):
    """H (n x n float32) <- (0 if reset else H) + alpha * X^T X, X tokens x n."""
    lib = load()
    _device_check(H)
    _rows_check(X)
    n = H.shape[0]
    if X.shape[1] != n or tuple(H.shape) != (n, n):
        raise ValueError("H must be n x n and X tokens x n")
    tokens = X.shape[0]
    dt = _dtype_code(X)
    need = lib.gptq_hessian_ws_bytes(n, tokens, dt)
    if ws is None:
        ws = _workspace(need, H.device)
    rc = lib.gptq_hessian_accumulate(_ptr(H), n, _ptr(X), dt, tokens, X.stride(0) if tokens else n,
                                     float(alpha), int(bool(reset)), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "gptq_hessian_accumulate")
    return H


def gptq_hessian_accumulate_noalloc(H, X, alpha: float = 2.0, reset: bool = False, stream=None):
    """As gptq_hessian_accumulate, with the library's static device scratch
    instead of a workspace (no allocation anywhere in the call)."""
    lib = load()
    _device_check(H)
    _rows_check(X)
    n = H.shape[0]
    if X.shape[1] != n or tuple(H.shape) != (n, n):
        raise ValueError("H must be n x n and X tokens x n")
    tokens = X.shape[0]
    rc = lib.gptq_hessian_accumulate_noalloc(_ptr(H), n, _ptr(X), _dtype_code(X), tokens,
                                             X.stride(0) if tokens else n, float(alpha), int(bool(reset)),
                                             _stream(stream))
    _check(rc, "gptq_hessian_accumulate_noalloc")
    return H


def gptq_hessian_pair_accumulate(H2, Xcat, alpha: float = 2.0, reset: bool = False, ws=None, stream=None):
    """H2 (2n x 2n float32): the Xq^T Xq and Xq^T Xf blocks of alpha Xcat^T Xcat
    for Xcat = [Xq | Xf] (tokens x 2n); the Xf^T Xf block is unspecified."""
    lib = load()
    _device_check(H2)
    _rows_check(Xcat)
    n2 = H2.shape[0]
    if n2 % 2 or Xcat.shape[1] != n2 or tuple(H2.shape) != (n2, n2):
        raise ValueError("H2 must be 2n x 2n and Xcat tokens x 2n")
    tokens = Xcat.shape[0]
    dt = _dtype_code(Xcat)
    if ws is None:
        ws = _workspace(lib.gptq_hessian_pair_ws_bytes(n2 // 2, tokens, dt), H2.device)
    rc = lib.gptq_hessian_pair_accumulate(_ptr(H2), n2 // 2, _ptr(Xcat), dt, tokens,
                                          Xcat.stride(0) if tokens else n2, float(alpha), int(bool(reset)),
                                          _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "gptq_hessian_pair_accumulate")
    return H2


def gptq_prepare_hinv(H, damp_rel: float = 0.01, act_order: bool = False, U=None, perm=None,
                      ws=None, stream=None):
    """Returns (U, perm): U^T U = (H[perm][:, perm] + lambda I)^{-1}, U upper."""
    torch = _torch()
    lib = load()
    _device_check(H)
    n = H.shape[0]
    if U is None:
        U = torch.empty((n, n), dtype=torch.float32, device=H.device)
    if perm is None:
        perm = torch.empty((n,), dtype=torch.int32, device=H.device)
    if ws is None:
        ws = _workspace(lib.gptq_prepare_ws_bytes(n), H.device)
    info = ctypes.c_int32(0)
    rc = lib.gptq_prepare_hinv(_ptr(H), n, float(damp_rel), int(bool(act_order)), _ptr(U), _ptr(perm),
                               ctypes.byref(info), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "gptq_prepare_hinv", info.value)
    return U, perm


def gptq_quantize_layer(W, U, perm=None, levels: int = 16, group_size: int = 0, block_size: int = 128,
                        want_row_loss: bool = True, want_g_idx: bool = True, want_wq: bool = False,
                        out=None, ws=None, stream=None):
    """Returns dict(codes (m x n uint8, original column order), scales (m x G),
    zeros (m x G uint8), g_idx (n int32) or None, row_loss (m) or None,
    Wq (m x n, W's dtype, dequantized) or None)."""
    torch = _torch()
    lib = load()
    _device_check(U, perm)
    _rows_check(W)
    m, n = W.shape
    if tuple(U.shape) != (n, n) or (perm is not None and perm.numel() != n):
        raise ValueError("U must be n x n and perm n long")
    G = 1 if group_size == 0 else -(-n // group_size)
    dev = W.device
    if out is None:
        out = dict(codes=torch.empty((m, n), dtype=torch.uint8, device=dev),
                   scales=torch.empty((m, G), dtype=torch.float32, device=dev),
                   zeros=torch.empty((m, G), dtype=torch.uint8, device=dev),
                   g_idx=torch.empty((n,), dtype=torch.int32, device=dev) if want_g_idx else None,
                   row_loss=torch.empty((m,), dtype=torch.float32, device=dev) if want_row_loss else None,
                   Wq=torch.empty((m, n), dtype=W.dtype, device=dev) if want_wq else None)
    for key in ("g_idx", "row_loss", "Wq"):
        out.setdefault(key, None)
    if out["Wq"] is not None and (out["Wq"].dtype != W.dtype or not out["Wq"].is_contiguous()):
        raise ValueError("Wq must be a contiguous m x n tensor of W's dtype")
    if ws is None:
        ws = _workspace(lib.gptq_quantize_ws_bytes(m, n, block_size), dev)
    rc = lib.gptq_quantize_layer(_ptr(W), _dtype_code(W), m, n, W.stride(0) if m else n, _ptr(U), _ptr(perm),
                                 int(levels), int(group_size), int(block_size), _ptr(out["codes"]),
                                 _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["g_idx"]),
                                 _ptr(out["row_loss"]), _ptr(out["Wq"]), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "gptq_quantize_layer")
    return out


def packed_words(n: int, bits: int) -> int:
    return -(-(n * bits) // 32)


def gptq_pack(codes, bits: int = 4, packed=None, stream=None):
    """packed (m x ceil(n*bits/32) int32 words: bit patterns of uint32) of
    codes in original column order."""
    torch = _torch()
    lib = load()
    _device_check(codes)
    m, n = codes.shape
    if packed is None:
        packed = torch.empty((m, packed_words(n, bits)), dtype=torch.int32, device=codes.device)
    rc = lib.gptq_pack(_ptr(codes), m, n, int(bits), _ptr(packed),
                       packed.stride(0) if m else packed_words(n, bits), _stream(stream))
    _check(rc, "gptq_pack")
    return packed


def gptq_dequant_gemv(packed, scales, zeros, X, n: int, bits: int, group_size: int = 0, g_idx=None,
                      Y=None, stream=None):
    """Y (batch x m float32) = X W^T with W^ read from the packed codes.

    packed: m x ld words (int32 bit patterns, as gptq_pack returns); scales
    m x G float32; zeros m x G uint8; X batch x n float16 (any leading
    dimension); g_idx n int32 or None (groups of group_size columns).
    """
    torch = _torch()
    lib = load()
    _rows_check(packed)
    _rows_check(X)
    _device_check(scales, zeros, g_idx)
    if X.dtype != torch.float16:
        raise ValueError("X must be float16")
    m = packed.shape[0]
    batch = X.shape[0]
    if X.shape[1] != n:
        raise ValueError("X must have n columns")
    if Y is None:
        Y = torch.empty((batch, m), dtype=torch.float32, device=X.device)
    else:
        _rows_check(Y)
    G = scales.shape[1] if scales.dim() == 2 else 1
    rc = lib.gptq_dequant_gemv(_ptr(packed), m, int(n), packed.stride(0), int(bits), _ptr(scales), _ptr(zeros),
                               int(G), int(group_size), _ptr(g_idx), _ptr(X), batch, X.stride(0), _ptr(Y),
                               Y.stride(0), _stream(stream))
    _check(rc, "gptq_dequant_gemv")
    return Y


def gptq_dequant_gemm(packed, scales, zeros, X, n: int, bits: int, group_size: int = 0, g_idx=None, Y=None,
                      stream=None):
    """Y (batch x m float32) = X W^T, any batch: on the matrix cores for
    groups of 0 or a multiple of 128 columns, else (act-order g_idx, narrower
    groups) on the VALU kernel, eight rows of X per pass."""
    torch = _torch()
    lib = load()
    _rows_check(packed)
    _rows_check(X)
    _device_check(scales, zeros, g_idx)
    if X.dtype != torch.float16:
        raise ValueError("X must be float16")
    m = packed.shape[0]
    batch = X.shape[0]
    if X.shape[1] != n:
        raise ValueError("X must have n columns")
    if Y is None:
        Y = torch.empty((batch, m), dtype=torch.float32, device=X.device)
    else:
        _rows_check(Y)
    G = scales.shape[1] if scales.dim() == 2 else 1
    rc = lib.gptq_dequant_gemm(_ptr(packed), m, int(n), packed.stride(0), int(bits), _ptr(scales), _ptr(zeros),
                               int(G), int(group_size), _ptr(g_idx), _ptr(X), batch, X.stride(0), _ptr(Y),
                               Y.stride(0), _stream(stream))
    _check(rc, "gptq_dequant_gemm")
    return Y


def gptq_asym_target(W, Hc, U, perm=None, Wt=None, ws=None, stream=None):
    """W' (m x n float32) = W Hc^T U^T U permuted back; Hc n x n (any leading dimension)."""
    torch = _torch()
    lib = load()
    _rows_check(W)
    _rows_check(Hc)
    _device_check(U, perm)
    m, n = W.shape
    if Wt is None:
        Wt = torch.empty((m, n), dtype=torch.float32, device=W.device)
    if ws is None:
        ws = _workspace(lib.gptq_asym_target_ws_bytes(m, n), W.device)
    rc = lib.gptq_asym_target(_ptr(W), _dtype_code(W), m, n, W.stride(0) if m else n, _ptr(Hc), Hc.stride(0),
                              _ptr(U), _ptr(perm), _ptr(Wt), Wt.stride(0) if m else n, _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "gptq_asym_target")
    return Wt


def gptaq_quantize_linear(W, Xq, Xf, levels: int = 16, group_size: int = 0, damp_rel: float = 0.01,
                          act_order: bool = False, block_size: int = 128, stream=None):
    """Asymmetric calibration for one layer: one paired Hessian call over [Xq | Xf],
    prepare on the Xq block, the target W', then the usual sweep and pack."""
    torch = _torch()
    n = W.shape[1]
    Xcat = torch.cat([Xq, Xf], dim=1)
    H2 = torch.empty((2 * n, 2 * n), dtype=torch.float32, device=W.device)
    gptq_hessian_pair_accumulate(H2, Xcat, 2.0, True, stream=stream)
    H = H2[:n, :n].contiguous()
    U, perm = gptq_prepare_hinv(H, damp_rel, act_order, stream=stream)
    p = perm if act_order else None
    Wt = gptq_asym_target(W, H2[:n, n:], U, p, stream=stream)
    q = gptq_quantize_layer(Wt, U, p, levels, group_size, block_size, stream=stream)
    packed = gptq_pack(q["codes"], bits_for_levels(levels), stream=stream)
    q.update(H=H, Hc=H2[:n, n:], U=U, perm=perm, Wt=Wt, packed=packed)
    return q


def gptq_lowrank_basis(H, Omega, iters: int = 10, L=None, ws=None, stream=None):
    """L (n x r float64, orthonormal columns) spanning H's top-r eigenvectors by
    subspace iteration from the caller's n x r float64 block Omega."""
    torch = _torch()
    lib = load()
    _rows_check(H)
    _device_check(Omega, L)
    n, r = Omega.shape
    if L is None:
        L = torch.empty((n, r), dtype=torch.float64, device=H.device)
    if ws is None:
        ws = _workspace(lib.gptq_lowrank_ws_bytes(0, n, r), H.device)
    rc = lib.gptq_lowrank_basis(_ptr(H), n, H.stride(0), r, _ptr(Omega), int(iters), _ptr(L), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "gptq_lowrank_basis")
    return L


def gptq_lowrank_hessian(H, L, H_L=None, K=None, ws=None, stream=None):
    """(H_L, K): H_L = H - H L M^{-1} L^T H (n x n float32), K = H L M^{-1}
    (n x r float64), M = L^T H L."""
    torch = _torch()
    lib = load()
    _rows_check(H)
    _device_check(L, K)
    n, r = L.shape
    if H_L is None:
        H_L = torch.empty((n, n), dtype=torch.float32, device=H.device)
    if K is None:
        K = torch.empty((n, r), dtype=torch.float64, device=H.device)
    if ws is None:
        ws = _workspace(lib.gptq_lowrank_ws_bytes(0, n, r), H.device)
    rc = lib.gptq_lowrank_hessian(_ptr(H), n, H.stride(0), _ptr(L), r, _ptr(H_L), H_L.stride(0), _ptr(K),
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "gptq_lowrank_hessian")
    return H_L, K


def gptq_lowrank_compensation(W, q, K, group_size: int = 0, R=None, ws=None, stream=None):
    """R (r x m float32) = K^T (W - W^)^T for gptq_quantize_layer's output q
    (codes in original column order; q["g_idx"] is used when present)."""
    torch = _torch()
    lib = load()
    _rows_check(W)
    g_idx = q.get("g_idx")
    _device_check(K, g_idx, q["codes"], q["scales"], q["zeros"])
    m, n = W.shape
    r = K.shape[1]
    if R is None:
        R = torch.empty((r, m), dtype=torch.float32, device=W.device)
    if ws is None:
        ws = _workspace(lib.gptq_lowrank_ws_bytes(m, n, r), W.device)
    rc = lib.gptq_lowrank_compensation(_ptr(W), _dtype_code(W), m, n, W.stride(0), _ptr(q["codes"]),
                                       _ptr(q["scales"]), _ptr(q["zeros"]), int(group_size), _ptr(g_idx), _ptr(K),
                                       r, _ptr(R), R.stride(0), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(stream))
    _check(rc, "gptq_lowrank_compensation")
    return R


def gptq_refine_codes(W, H, q, levels: int, group_size: int = 0, sweeps: int = 1, L=None, R=None, codes=None,
                      ws=None, stream=None):
    """Fixed-grid refinement of q's codes (coordinate descent on the error
    1/2 d H d^T, d = W - R^T L^T - W^, grid q["scales"] / q["zeros"] /
    q["g_idx"] held fixed).  H is the undamped calibration Hessian.  The
    refined codes go to `codes` (default: a copy of q["codes"]).  Returns
    (codes, moves), moves an int64 device tensor with the number of codes
    changed in each sweep."""
    torch = _torch()
    lib = load()
    _rows_check(W)
    _rows_check(H)
    g_idx = q.get("g_idx")
    _device_check(L, R, g_idx, q["codes"], q["scales"], q["zeros"], codes)
    m, n = W.shape
    r = 0 if L is None else L.shape[1]
    if codes is None:
        codes = q["codes"].clone()
    moves = torch.zeros(max(1, int(sweeps)), dtype=torch.int64, device=W.device)
    if ws is None:
        ws = _workspace(lib.gptq_refine_ws_bytes(m, n), W.device)
    rc = lib.gptq_refine_codes(_ptr(W), _dtype_code(W), m, n, W.stride(0), _ptr(H), H.stride(0), _ptr(L), _ptr(R),
                               r, 0 if R is None else R.stride(0), _ptr(q["scales"]), _ptr(q["zeros"]),
                               int(group_size), _ptr(g_idx), int(levels), int(sweeps), _ptr(codes), _ptr(moves),
                               _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "gptq_refine_codes")
    return codes, moves[:int(sweeps)]


def gptq_lora_refine(W, q, levels: int, group_size: int = 0, rounds: int = 1, sweeps: int = 1,
                     joint: bool = True, stream=None):
    """Alternates the fixed-grid refinement with R = R*(codes) for a layer
    from gptq_lora_quantize_linear (q holds H, H_L, L, K, R, the grid and the
    codes).  joint=True refines on H_L (every move optimal over the code and
    R together); joint=False holds the current R fixed and refines on H.
    Updates q["codes"], q["R"] and q["packed"]; returns the moves of each
    round (int64 device tensor, rounds x sweeps)."""
    torch = _torch()
    ws = _workspace(load().gptq_refine_ws_bytes(W.shape[0], W.shape[1]), W.device)
    per_round = []
    for _ in range(int(rounds)):
        if joint:
            codes, moves = gptq_refine_codes(W, q["H_L"], q, levels, group_size, sweeps, codes=q["codes"], ws=ws,
                                             stream=stream)
        else:
            codes, moves = gptq_refine_codes(W, q["H"], q, levels, group_size, sweeps, L=q["L"], R=q["R"],
                                             codes=q["codes"], ws=ws, stream=stream)
        q["codes"] = codes
        q["R"] = gptq_lowrank_compensation(W, q, q["K"], group_size, R=q["R"], stream=stream)
        per_round.append(moves)
    q["packed"] = gptq_pack(q["codes"], bits_for_levels(levels), stream=stream)
    return torch.stack(per_round) if per_round else torch.zeros((0, int(sweeps)), dtype=torch.int64)


def gptq_lora_quantize_linear(W, X=None, H=None, rank: int = 16, levels: int = 16, group_size: int = 0,
                              damp_rel: float = 0.01, act_order: bool = False, block_size: int = 128,
                              iters: int = 10, seed: int = 0, Omega=None, stream=None):
    """GPTQ with the low-rank correction for one layer: H, L = V_r (subspace
    iteration from Omega, by default a seeded standard normal n x r block),
    H_L and K, then prepare/quantize/pack on H_L and finally R."""
    torch = _torch()
    n = W.shape[1]
    if H is None:
        H = torch.empty((n, n), dtype=torch.float32, device=W.device)
        gptq_hessian_accumulate(H, X, 2.0, True, stream=stream)
    if Omega is None:
        gen = torch.Generator(device=W.device).manual_seed(int(seed))
        Omega = torch.randn((n, rank), generator=gen, device=W.device, dtype=torch.float64)
    L = gptq_lowrank_basis(H, Omega, iters, stream=stream)
    H_L, K = gptq_lowrank_hessian(H, L, stream=stream)
    U, perm = gptq_prepare_hinv(H_L, damp_rel, act_order, stream=stream)
    p = perm if act_order else None
    q = gptq_quantize_layer(W, U, p, levels, group_size, block_size, stream=stream)
    packed = gptq_pack(q["codes"], bits_for_levels(levels), stream=stream)
    R = gptq_lowrank_compensation(W, q, K, group_size, stream=stream)
    q.update(H=H, L=L, H_L=H_L, K=K, U=U, perm=perm, packed=packed, R=R)
    return q


def bits_for_levels(levels: int) -> int:
    return {3: 2, 4: 2, 8: 3, 16: 4}[int(levels)]


def gptq_quantize_linear(W, X=None, H=None, levels: int = 16, group_size: int = 0,
                         damp_rel: float = 0.01, act_order: bool = False, block_size: int = 128,
                         stream=None):
    """All four calls in order for one layer (convenience wrapper)."""
    torch = _torch()
    n = W.shape[1]
    if H is None:
        H = torch.empty((n, n), dtype=torch.float32, device=W.device)
        gptq_hessian_accumulate(H, X, 2.0, True, stream=stream)
    U, perm = gptq_prepare_hinv(H, damp_rel, act_order, stream=stream)
    q = gptq_quantize_layer(W, U, perm if act_order else None, levels, group_size, block_size,
                            stream=stream)
    packed = gptq_pack(q["codes"], bits_for_levels(levels), stream=stream)
    q.update(H=H, U=U, perm=perm, packed=packed)
    return q
