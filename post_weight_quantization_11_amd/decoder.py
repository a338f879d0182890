"""Sequential quantization of a Llama-shaped decoder (the whole-model pass).

Wiki "GPTQ", "Technical Approach": the method processes layers one after
another; GPTQ knowledge note, "How It Works": each linear layer's Hessian
comes from that layer's recorded inputs.  Here every block's calibration
inputs are produced by the blocks before it *after* they were quantized, and
within a block the attention output projection sees the quantized q/k/v, the
MLP the quantized attention.  q, k and v read the same normalised input, so
they share one Hessian and one factor U; gate and up likewise.

This module is a harness around the library: the decoder's forward pass
(RMSNorm, rotary attention, SwiGLU MLP) uses torch operations, every
quantizer step runs through the C ABI (gptq_hessian_accumulate,
gptq_prepare_hinv, gptq_quantize_layer, gptq_pack).  Weights are random
(seeded); there is no trained model.
"""
from __future__ import annotations

import dataclasses
import math

from . import _lib

LINEARS = ("q", "k", "v", "o", "gate", "up", "down")


@dataclasses.dataclass(frozen=True)
class DecoderShape:
    d_model: int = 4096
    d_ff: int = 11008
    n_heads: int = 32
    n_blocks: int = 32
    rope_base: float = 10000.0
    eps: float = 1e-6


LLAMA_7B = DecoderShape()


def linear_shapes(shape: DecoderShape):
    d, f = shape.d_model, shape.d_ff
    return {"q": (d, d), "k": (d, d), "v": (d, d), "o": (d, d), "gate": (f, d), "up": (f, d), "down": (d, f)}


def random_blocks(shape: DecoderShape, seed: int, device, dtype, w_std: float = 0.02):
    """Seeded N(0, w_std^2) weights for every block, stored in `dtype`."""
    torch = _lib._torch()
    gen = torch.Generator(device=device).manual_seed(int(seed))
    blocks = []
    for _ in range(shape.n_blocks):
        blk = {}
        for name, (rows, cols) in linear_shapes(shape).items():
            blk[name] = (torch.randn((rows, cols), generator=gen, device=device) * w_std).to(dtype)
        blocks.append(blk)
    return blocks


# ---------------------------------------------------------------------------
# Forward pass pieces (torch; `x` is tokens x features, tokens = seqs * seq_len).
# ---------------------------------------------------------------------------
def rms_norm(x, eps: float):
    """x / sqrt(mean(x^2) + eps) per token (unit gain)."""
    torch = _lib._torch()
    return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + eps)


def rope(x, base: float):
    """Rotary position embedding on (seqs, seq_len, heads, head_dim): the
    first and second halves of each head form the rotated pairs."""
    torch = _lib._torch()
    seq_len, hd = x.shape[1], x.shape[3]
    half = hd // 2
    inv = base ** (-torch.arange(half, device=x.device, dtype=x.dtype) * 2.0 / hd)
    ang = torch.arange(seq_len, device=x.device, dtype=x.dtype)[:, None] * inv[None, :]
    cos, sin = ang.cos()[None, :, None, :], ang.sin()[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat((x1 * cos - x2 * sin, x1 * sin + x2 * cos), dim=-1)


def attention(h, Wq, Wk, Wv, shape: DecoderShape, seqs: int, seq_len: int, chunk: int = 4):
    """Causal multi-head attention output (before the o projection), in the
    dtype of h; scores and softmax in float32 (float64 if h is float64)."""
    torch = _lib._torch()
    H, D = shape.n_heads, shape.d_model // shape.n_heads
    acc = torch.float64 if h.dtype == torch.float64 else torch.float32
    q = (h @ Wq.T).view(seqs, seq_len, H, D).to(acc)
    k = (h @ Wk.T).view(seqs, seq_len, H, D).to(acc)
    v = (h @ Wv.T).view(seqs, seq_len, H, D).to(acc)
    q = rope(q, shape.rope_base).permute(0, 2, 1, 3).contiguous()
    k = rope(k, shape.rope_base).permute(0, 2, 3, 1).contiguous()     # keys transposed, materialised
    v = v.permute(0, 2, 1, 3).contiguous()
    mask = torch.ones((seq_len, seq_len), dtype=torch.bool, device=h.device).tril()
    out = torch.empty((seqs, H, seq_len, D), dtype=acc, device=h.device)
    for s0 in range(0, seqs, chunk):
        sc = torch.matmul(q[s0:s0 + chunk], k[s0:s0 + chunk]) / math.sqrt(D)
        sc = sc.masked_fill(~mask, float("-inf")).softmax(-1)
        out[s0:s0 + chunk] = torch.matmul(sc, v[s0:s0 + chunk])
    return out.permute(0, 2, 1, 3).reshape(seqs * seq_len, H * D).to(h.dtype)


def dequantize(q, group_size: int, dtype):
    """W^ = s_g (c - z_g) in original column order, formed in float64 (exact:
    a float32 scale times a small integer) from the codes and g_idx."""
    torch = _lib._torch()
    codes = q["codes"].to(torch.float64)
    n = codes.shape[1]
    if q.get("g_idx") is not None:
        gi = q["g_idx"].long()
    else:
        gi = torch.zeros(n, dtype=torch.long, device=codes.device) if group_size == 0 else \
            torch.arange(n, device=codes.device) // group_size
    w = q["scales"].to(torch.float64)[:, gi] * (codes - q["zeros"].to(torch.float64)[:, gi])
    return w.to(dtype)


# ---------------------------------------------------------------------------
# The sequential pass.
# ---------------------------------------------------------------------------
def quantize_decoder(blocks, X, shape: DecoderShape, seqs: int, seq_len: int, levels: int = 4,
                     group_size: int = 64, act_order: bool = False, damp_rel: float = 0.01,
                     h_dtype=None, timer=None, keep_inputs: bool = False):
    """Quantizes every linear layer of every block in order.

    X: tokens x d_model calibration inputs of the first block (the dtype the
    forward pass runs in).  h_dtype: dtype in which layer inputs are handed to
    gptq_hessian_accumulate (float32, float16 or bfloat16; default: X's dtype,
    float32 if X is float64).  timer(stage) -> context manager, optional.

    Returns (X_out, results): results[b][name] = dict(codes (original column
    order), scales, zeros, g_idx, row_loss, Wq (or None), perm, packed) for
    block b; with keep_inputs also the layer input as handed to the Hessian
    call ("X_in"), the Hessian ("H") and the factor ("U").
    """
    torch = _lib._torch()
    if h_dtype is None:
        h_dtype = torch.float32 if X.dtype == torch.float64 else X.dtype
    bits = _lib.bits_for_levels(levels)
    dev = X.device
    cdt = X.dtype

    class _Null:
        def __enter__(self):
            return self

        def __exit__(self, *a):
            return False

    def stage(name):
        return timer(name) if timer is not None else _Null()

    kept = {}

    def factor(inp):
        n = inp.shape[1]
        H = torch.empty((n, n), dtype=torch.float32, device=dev)
        X_in = inp.to(h_dtype).contiguous()
        with stage("hessian"):
            _lib.gptq_hessian_accumulate(H, X_in, 2.0, True)
        with stage("prepare"):
            U, perm = _lib.gptq_prepare_hinv(H, damp_rel, act_order)
        if keep_inputs:
            kept.update(X_in=X_in, H=H, U=U)
        return U, (perm if act_order else None)

    # The forward runs on the library's dequantized weights (Wq, in W's dtype)
    # when it runs in that dtype; a float64 forward (validation) forms them
    # exactly from the codes.
    def quant(W, U, perm):
        exact = cdt != W.dtype
        with stage("quantize"):
            q = _lib.gptq_quantize_layer(W, U, perm, levels, group_size, 128, want_wq=not exact)
        with stage("pack"):
            packed = _lib.gptq_pack(q["codes"], bits)
        q.update(perm=perm, packed=packed, **kept)
        with stage("forward"):
            What = dequantize(q, group_size, cdt) if exact else q["Wq"]
        return q, What

    results = []
    for blk in blocks:
        res = {}
        Wq = {}
        with stage("forward"):
            h = rms_norm(X, shape.eps)
        U, perm = factor(h)                                  # shared by q, k, v
        for name in ("q", "k", "v"):
            res[name], Wq[name] = quant(blk[name], U, perm)
        with stage("forward"):
            a = attention(h, Wq["q"], Wq["k"], Wq["v"], shape, seqs, seq_len)
        U, perm = factor(a)
        res["o"], Wq["o"] = quant(blk["o"], U, perm)
        with stage("forward"):
            X = X + a @ Wq["o"].T
            h2 = rms_norm(X, shape.eps)
        U, perm = factor(h2)                                 # shared by gate, up
        for name in ("gate", "up"):
            res[name], Wq[name] = quant(blk[name], U, perm)
        with stage("forward"):
            mm = torch.nn.functional.silu(h2 @ Wq["gate"].T) * (h2 @ Wq["up"].T)
        U, perm = factor(mm)
        res["down"], Wq["down"] = quant(blk["down"], U, perm)
        with stage("forward"):
            X = X + mm @ Wq["down"].T
        results.append(res)
    return X, results
