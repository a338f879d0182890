"""Plain CPU oracle of the sequential whole-decoder quantization pass.

TEST INFRASTRUCTURE ONLY (like the rest of this package): numpy float64,
nothing on the product path imports it.

Wiki "GPTQ", "Technical Approach": layers are processed one after another;
GPTQ knowledge note, "How It Works": a layer's Hessian is H = 2 X X^T over
that layer's recorded inputs.  Each block's inputs come from the blocks
before it after they were quantized; inside a block, q/k/v share the Hessian
of the normalised block input, o sees the attention computed with quantized
q/k/v, gate/up share the Hessian of the normalised residual stream, down sees
SwiGLU of quantized gate/up.  The decoder is Llama-shaped: RMSNorm with unit
gain, rotary embeddings (first and second halves of each head rotated
together, base 10000), causal softmax attention, SwiGLU MLP.  These are the
plainest readings; the pages name the protocol, not an architecture.

Each layer input is rounded to float32 before its Hessian is formed (the
precision in which the GPU pass hands it to gptq_hessian_accumulate).
"""
from __future__ import annotations

import numpy as np

from .gptq_oracle import (act_order_perm, damp_and_permute, dequantize, gptq_quantize, hessian,
                          inverse_cholesky_upper)

F64 = np.float64


def rms_norm(x, eps=1e-6):
    x = np.asarray(x, dtype=F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, base=10000.0):
    """x: (seqs, seq_len, heads, head_dim)."""
    seq_len, hd = x.shape[1], x.shape[3]
    half = hd // 2
    inv = base ** (-np.arange(half, dtype=F64) * 2.0 / hd)
    ang = np.arange(seq_len, dtype=F64)[:, None] * inv[None, :]
    cos, sin = np.cos(ang)[None, :, None, :], np.sin(ang)[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate((x1 * cos - x2 * sin, x1 * sin + x2 * cos), axis=-1)


def attention(h, Wq, Wk, Wv, n_heads, seqs, seq_len, base=10000.0):
    d = h.shape[1]
    D = d // n_heads
    q = rope((h @ Wq.T).reshape(seqs, seq_len, n_heads, D), base)
    k = rope((h @ Wk.T).reshape(seqs, seq_len, n_heads, D), base)
    v = (h @ Wv.T).reshape(seqs, seq_len, n_heads, D)
    out = np.zeros((seqs, seq_len, n_heads, D), dtype=F64)
    for s in range(seqs):
        for hh in range(n_heads):
            sc = q[s, :, hh, :] @ k[s, :, hh, :].T / np.sqrt(D)
            sc = np.where(np.tril(np.ones((seq_len, seq_len), dtype=bool)), sc, -np.inf)
            sc = np.exp(sc - sc.max(axis=1, keepdims=True))
            sc /= sc.sum(axis=1, keepdims=True)
            out[s, :, hh, :] = sc @ v[s, :, hh, :]
    return out.reshape(seqs * seq_len, d)


def silu(x):
    return x / (1.0 + np.exp(-x))


def quantize_decoder(blocks, X, n_heads, seqs, seq_len, levels=4, group_size=64, act_order=False,
                     damp_rel=0.01, block_size=128, eps=1e-6):
    """blocks: list of dicts name -> W (numpy, out x in); X: tokens x d (float64).

    Returns (X_out, results): results[b][name] = dict of gptq_quantize's
    outputs plus perm, U, the layer's W (float64) and its dequantization.
    """
    X = np.asarray(X, dtype=F64)
    results = []

    def factor(inp):
        H = hessian(np.asarray(inp, dtype=np.float32).astype(F64))
        perm = act_order_perm(H) if act_order else np.arange(H.shape[0])
        Hd, _ = damp_and_permute(H, perm, damp_rel)
        return inverse_cholesky_upper(Hd), perm

    def quant(W, U, perm):
        W = np.asarray(W, dtype=F64)
        r = gptq_quantize(W, U, perm, levels, group_size, block_size)
        r.update(U=U, perm=perm, W=W)
        r["What"] = dequantize(r)
        return r

    for blk in blocks:
        res = {}
        h = rms_norm(X, eps)
        U, perm = factor(h)
        for name in ("q", "k", "v"):
            res[name] = quant(blk[name], U, perm)
        a = attention(h, res["q"]["What"], res["k"]["What"], res["v"]["What"], n_heads, seqs, seq_len)
        U, perm = factor(a)
        res["o"] = quant(blk["o"], U, perm)
        X = X + a @ res["o"]["What"].T
        h2 = rms_norm(X, eps)
        U, perm = factor(h2)
        for name in ("gate", "up"):
            res[name] = quant(blk[name], U, perm)
        mm = silu(h2 @ res["gate"]["What"].T) * (h2 @ res["up"]["What"].T)
        U, perm = factor(mm)
        res["down"] = quant(blk["down"], U, perm)
        X = X + mm @ res["down"]["What"].T
        results.append(res)
    return X, results
