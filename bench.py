"""Benchmark: one GPTQ layer quantization per step on one MI355X.

A step runs the whole path on inputs already resident in HBM:
  gptq_hessian_accumulate (all calibration tokens, reset)
  gptq_prepare_hinv       (damping, act-order, U)
  gptq_quantize_layer     (column sweep + lazy block updates)
  gptq_pack               (un-permute + pack, g_idx)
Default workload: Llama-7B-shaped attention projection, W 4096 x 4096 bf16,
262144 calibration tokens (128 x 2048) bf16 with Student-t(4) channel
scales, 4-bit asymmetric, group size 128, block 128, damping 1%.

Prints one JSON line: columns/s of the whole step, per-stage times and
roofline fractions, the dominant kernel's roofline record and the CPU
oracle's time on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
                       [--no-cpu] [--copy-calibration]

`--decoder` instead times the sequential whole-decoder pass (post_weight_
quantization_11_amd.decoder): 32 Llama-7B-shaped blocks of random bf16
weights, 128 x 2048 calibration tokens fed through the already-quantized
blocks, 2-bit g64 (`--levels 3` for the ternary variant); one JSON line with
the total time and its split over Hessian / prepare / quantize / pack /
forward (HIP events on the stream).

`--gptaq` instead times the asymmetric-calibration variant on the 4096 x 4096
layer (Xq = the quantized model's inputs, here X plus 5% noise; Xf = X):
one paired Hessian call over [Xq | Xf] (the Xf^T Xf tiles skipped), prepare,
the target W' (three float32
matrix products), sweep, pack; one JSON line with the per-stage times.

`--lora` instead times GPTQ with the low-rank correction (GPTQ-intrinsic
LoRA reading) on the same 4096 x 4096 layer: Hessian, the rank-`--rank`
basis (subspace iteration, `--lora-iters` steps), the augmented Hessian H_L,
prepare / sweep / pack on H_L and the compensation R; one JSON line with the
per-stage times and their float64 roofline fractions.

`--gemv` instead times the packed-weight decode product gptq_dequant_gemv
(Y = X W^T from the packed codes) on the 175B-class fc1 layer, 49152 x
12288 4-bit per-row, batch `--gemv-batch` (default 1), and prints its own
JSON line with the HBM roofline record.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "GPTQ per-layer quant time (ms), columns/s, % MFMA peak + HBM GB/s per stage"

# MI355X published peaks.
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_F64_TFLOPS = 78.6
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_device(st):
    import torch
    if st.dtype == "bf16":
        return torch.from_numpy(st.raw.view(np.int16)).view(torch.bfloat16).cuda()
    if st.dtype == "f16":
        return torch.from_numpy(st.raw).cuda()
    return torch.from_numpy(st.raw).cuda()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hessian_attn_proj_4096_traffic.md")
TRAFFIC_SOURCES = [os.path.join(ROOT, "post_weight_quantization_11_amd", "csrc", f) for f in ("hessian.hip", "common.h")]


def measured_traffic(config):
    """HBM bytes per Hessian call from the committed FETCH_SIZE/WRITE_SIZE
    profile of the 4096-wide workload, or None when that profile was taken on
    other kernel sources than the ones built here (or for other workloads)."""
    import hashlib
    if config != 2 or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and line.split(":")[0].strip() in ("traffic_bytes_per_launch", "sources_sha256"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    if fields.get("sources_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def bits_of(levels):
    return {3: 2, 4: 2, 8: 3, 16: 4}[levels]


def cpu_baseline(L, X, cfg, n, m, tokens_total):
    """Times the CPU oracle on a bounded sample of the same workload and
    scales each stage to the full workload.  Returns the record."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    except Exception:  # pragma: no cover
        threads, blas = os.cpu_count() or 1, "unknown"
    t_sample = min(tokens_total, 32768)
    m_sample = min(m, 1024)
    Xs = wl.Stored(X.raw[:t_sample], X.dtype).f32 if X is not None else L.x_all(t_sample).f32
    t0 = time.perf_counter()
    H = oracle.hessian(Xs)
    t_h = (time.perf_counter() - t0) * (tokens_total / t_sample)
    H = H * (tokens_total / t_sample)          # same scale as the full Hessian
    t0 = time.perf_counter()
    perm = oracle.act_order_perm(H) if cfg.act_order else np.arange(n)
    Hd, _ = oracle.damp_and_permute(H, perm, cfg.damp_rel)
    U = oracle.inverse_cholesky_upper(Hd)
    t_p = time.perf_counter() - t0
    W64 = L.W.f32[:m_sample].astype(np.float64)
    t0 = time.perf_counter()
    res = oracle.gptq_quantize(W64, U, perm, cfg.levels, cfg.group_size, cfg.block_size)
    t_q = (time.perf_counter() - t0) * (m / m_sample)
    t0 = time.perf_counter()
    oracle.pack_codes(oracle.unpermute_codes(res["codes"], perm).astype(np.int64), bits_of(cfg.levels))
    t_k = (time.perf_counter() - t0) * (m / m_sample)
    total = t_h + t_p + t_q + t_k
    return {
        "value": n / total,
        "unit": "columns/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"Hessian on {t_sample} of {tokens_total} tokens (x{tokens_total / t_sample:g}); "
                   f"damp/act-order/U at full n={n}; sweep and pack on {m_sample} of {m} rows with the "
                   f"full U (x{m / m_sample:g}, rows are independent); numpy float64, BLAS={blas}"),
        "stage_s": {"hessian": t_h, "prepare": t_p, "quantize": t_q, "pack": t_k},
        "ms_per_layer": total * 1e3,
        "host": platform.processor() or platform.machine(),
        "os_cpu_count": os.cpu_count(),
    }


def bench_decoder(args):
    """Sequential whole-decoder pass, Llama-7B shapes, random weights."""
    import contextlib
    import torch
    from post_weight_quantization_11_amd import decoder as dec
    shape = dataclasses_replace(dec.LLAMA_7B, n_blocks=args.decoder_blocks)
    seqs, S = args.decoder_seqs, args.decoder_seq_len
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    blocks = dec.random_blocks(shape, seed=2024, device="cuda", dtype=torch.bfloat16)
    gen = torch.Generator(device="cuda").manual_seed(7)
    X0 = torch.randn((seqs * S, shape.d_model), device="cuda", generator=gen).to(torch.bfloat16)
    torch.cuda.synchronize()
    log(f"decoder weights and inputs generated in {time.perf_counter() - t0:.1f}s")
    stream = torch.cuda.current_stream()
    marks = []

    @contextlib.contextmanager
    def timer(name):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        yield
        e1.record(stream)
        marks.append((name, e0, e1))

    torch.cuda.synchronize()
    t1 = time.perf_counter()
    Xout, res = dec.quantize_decoder(blocks, X0, shape, seqs, S, levels=args.levels, group_size=args.group_size,
                                     act_order=False, timer=timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    split = {}
    for name, e0, e1 in marks:
        split[name] = split.get(name, 0.0) + e0.elapsed_time(e1) / 1e3
    nlayers = len(res) * len(dec.LINEARS)
    finite = bool(torch.isfinite(Xout.float()).all().item())
    rec = {
        "metric": "whole-decoder GPTQ pass time (s), layers/s",
        "value": wall,
        "unit": "s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 0,
        "ms_per_step": wall * 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 forward, f32/f64 quantizer",
        "data": "synthetic",
        "config": {"workload": "Llama-7B-shaped decoder pass", "blocks": shape.n_blocks, "d_model": shape.d_model,
                   "d_ff": shape.d_ff, "heads": shape.n_heads, "seqs": seqs, "seq_len": S, "levels": args.levels,
                   "group_size": args.group_size, "parallelism": "1 GPU"},
        "layers": nlayers,
        "layers_per_s": nlayers / wall,
        "stage_s": split,
        "quantizer_s": sum(v for k, v in split.items() if k != "forward"),
        "sanity": {"finite_output": finite},
    }
    print(json.dumps(rec), flush=True)


def bench_gptaq(args):
    """Asymmetric calibration on the Llama-7B attention projection (4096 x 4096, 262144 tokens)."""
    import torch
    import post_weight_quantization_11_amd as g
    cfg = wl.WORKLOADS[2]
    m, n, N = 4096, 4096, cfg.tokens
    torch.cuda.set_device(0)
    L = wl.workload_layer(2, 0)
    X = to_device(L.x_all())
    Wd = to_device(L.W)
    gen = torch.Generator(device="cuda").manual_seed(5)
    Xcat = torch.empty((N, 2 * n), dtype=torch.bfloat16, device="cuda")
    Xcat[:, n:] = X
    Xcat[:, :n] = (X.float() * (1.0 + 0.05 * torch.randn(X.shape, device="cuda", generator=gen))).to(torch.bfloat16)
    del X
    H2 = torch.empty((2 * n, 2 * n), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    names = ["hessian", "prepare", "target", "quantize", "pack"]

    def step(ev=None):
        mark = (lambda i: ev[i].record(stream)) if ev else (lambda i: None)
        mark(0)
        g.gptq_hessian_pair_accumulate(H2, Xcat, 2.0, True)
        mark(1)
        H = H2[:n, :n].contiguous()
        U, perm = g.gptq_prepare_hinv(H, cfg.damp_rel, False)
        mark(2)
        Wt = g.gptq_asym_target(Wd, H2[:n, n:], U, None)
        mark(3)
        q = g.gptq_quantize_layer(Wt, U, None, cfg.levels, cfg.group_size, cfg.block_size)
        mark(4)
        g.gptq_pack(q["codes"], None, bits_of(cfg.levels), cfg.group_size)
        mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    st = {k: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, k in enumerate(names)}
    tflops_t = 3 * 2.0 * m * n * n / (st["target"] * 1e-3) / 1e12
    rec = {
        "metric": "GPTAQ per-layer time (ms), asymmetric calibration",
        "value": wall * 1e3,
        "unit": "ms per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs, f32/f64 quantizer",
        "data": "synthetic",
        "config": {"workload": cfg.name + ", asymmetric calibration (Xq = X with 5% noise)", "m": m, "n": n,
                   "tokens": N, "levels": cfg.levels, "group_size": cfg.group_size, "parallelism": "1 GPU"},
        "stage_ms": st,
        "target_roofline": {"bound": "mfma", "achieved": tflops_t, "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                            "frac": tflops_t / PEAK_F32_TFLOPS,
                            "algorithmic": "3 m n^2 multiply-adds (W Hc^T, x U^T, x U)"},
    }
    print(json.dumps(rec), flush=True)


def bench_lora(args):
    """Low-rank corrected GPTQ on the Llama-7B attention projection (4096 x 4096, 262144 tokens)."""
    import torch
    import post_weight_quantization_11_amd as g
    cfg = wl.WORKLOADS[2]
    m, n, N, r, iters = 4096, 4096, cfg.tokens, args.rank, args.lora_iters
    torch.cuda.set_device(0)
    L = wl.workload_layer(2, 0)
    X = to_device(L.x_all())
    Wd = to_device(L.W)
    H = torch.empty((n, n), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(7)
    Omega = torch.randn((n, r), generator=gen, device="cuda", dtype=torch.float64)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    names = ["hessian", "basis", "lowrank_hessian", "prepare", "quantize", "pack", "compensation"]
    out = {}

    def step(ev=None):
        mark = (lambda i: ev[i].record(stream)) if ev else (lambda i: None)
        mark(0)
        g.gptq_hessian_accumulate(H, X, 2.0, True)
        mark(1)
        Lb = g.gptq_lowrank_basis(H, Omega, iters)
        mark(2)
        HL, K = g.gptq_lowrank_hessian(H, Lb)
        mark(3)
        U, perm = g.gptq_prepare_hinv(HL, cfg.damp_rel, False)
        mark(4)
        q = g.gptq_quantize_layer(Wd, U, None, cfg.levels, cfg.group_size, cfg.block_size)
        mark(5)
        g.gptq_pack(q["codes"], None, bits_of(cfg.levels), cfg.group_size)
        mark(6)
        R = g.gptq_lowrank_compensation(Wd, q, K, None, cfg.group_size)
        mark(7)
        out.update(q=q, R=R, L=Lb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    st = {k: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, k in enumerate(names)}
    # Algorithmic float64 flops: H Q per iteration (2 n^2 r) plus the Cholesky-QR
    # Gram and triangular products (4 n r^2 per pass, iters + 2 passes); H L and
    # the downdate (4 n^2 r) plus L^T H L, C^{-T} and C^{-1} (6 n r^2); R (2 m n r).
    fl = {"basis": iters * 2.0 * n * n * r + (iters + 2) * 4.0 * n * r * r,
          "lowrank_hessian": 4.0 * n * n * r + 6.0 * n * r * r,
          "compensation": 2.0 * m * n * r}
    roof = {k: {"ms": st[k], "tflops": fl[k] / (st[k] * 1e-3) / 1e12,
                "frac": fl[k] / (st[k] * 1e-3) / 1e12 / PEAK_F64_TFLOPS} for k in fl}
    Lh = out["L"]
    orth = float((Lh.T @ Lh - torch.eye(r, dtype=torch.float64, device="cuda")).abs().max())
    rec = {
        "metric": "GPTQ with low-rank correction, per-layer time (ms)",
        "value": wall * 1e3,
        "unit": "ms per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs, f64 low-rank stages, f32/f64 quantizer",
        "data": "synthetic",
        "config": {"workload": cfg.name + f", rank-{r} correction (L = V_r by {iters} subspace iterations)",
                   "m": m, "n": n, "tokens": N, "rank": r, "iters": iters, "levels": cfg.levels,
                   "group_size": cfg.group_size, "parallelism": "1 GPU"},
        "stage_ms": st,
        "lowrank_roofline": {"bound": "f64 VALU", "peak": PEAK_F64_TFLOPS, "unit": "TFLOP/s", "stages": roof},
        "sanity": {"L_orthonormal_maxerr": orth, "R_finite": bool(torch.isfinite(out["R"]).all())},
    }
    print(json.dumps(rec), flush=True)


def dataclasses_replace(obj, **kw):
    import dataclasses
    return dataclasses.replace(obj, **kw)


def bench_gemv(args):
    """Decode product on the 175B-class fc1 layer (49152 x 12288, 4-bit per-row)."""
    import torch
    import post_weight_quantization_11_amd as g
    m, n, bits, batch = 49152, 12288, 4, args.gemv_batch
    torch.cuda.set_device(0)
    gen = torch.Generator(device="cuda").manual_seed(2023)
    nw = g.packed_words(n, bits)
    packed = torch.randint(-2**31, 2**31 - 1, (m, nw), dtype=torch.int32, device="cuda", generator=gen)
    scales = torch.rand((m, 1), device="cuda", generator=gen) * 0.015 + 0.005
    zeros = torch.randint(0, 1 << bits, (m, 1), dtype=torch.uint8, device="cuda", generator=gen)
    X = torch.randn((batch, n), device="cuda", generator=gen).half()
    Y = torch.empty((batch, m), device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        g.gptq_dequant_gemv(packed, scales, zeros, X, n, bits, Y=Y)
    torch.cuda.synchronize()
    # HIP events around each launch on the launching stream: the kernel's own duration.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        g.gptq_dequant_gemv(packed, scales, zeros, X, n, bits, Y=Y)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3
    nbytes = float(m) * nw * 4 + m * 5 + batch * n * 2 + batch * m * 4
    rec = {
        "metric": "packed-weight decode product time (us), HBM GB/s",
        "value": us,
        "unit": "us per call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 x 4-bit codes, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "175B-class fc1 decode product", "m": m, "n": n, "bits": bits, "group_size": 0,
                   "batch": batch, "parallelism": "1 GPU"},
        "roofline": {
            "kernel": ("dequant_gemv_kernel<4> (VALU dot2)" if batch <= 2 else "dequant_mfma_kernel<4> (matrix cores)")
                      + " via gptq_dequant_gemv, HIP events around each launch",
            "bound": "hbm",
            "achieved": nbytes / (us * 1e-6) / 1e9,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "traffic": None,
            "algorithmic": f"packed words + scales/zeros + X + Y = {nbytes:.4g} bytes per launch",
        },
    }
    if not args.no_cpu:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        rows = 8192
        w = packed[:rows].cpu().numpy().view(np.uint32)
        s_, z_ = scales[:rows].cpu().numpy(), zeros[:rows].cpu().numpy()
        x = X.cpu().numpy().astype(np.float64)
        t1 = time.perf_counter()
        oracle.dequant_matmul(w, n, bits, s_, z_, np.zeros(n, dtype=np.int32), x)
        cpu = time.perf_counter() - t1
        rec["cpu_baseline"] = {"value": cpu * (m / rows) * 1e6, "unit": "us per call", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"oracle.dequant_matmul on {rows} of the {m} rows, scaled by {m // rows}"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--gemv", action="store_true", help="time the packed-weight decode product instead")
    ap.add_argument("--gemv-batch", type=int, default=1)
    ap.add_argument("--decoder", action="store_true", help="time the whole-decoder pass instead")
    ap.add_argument("--decoder-blocks", type=int, default=32)
    ap.add_argument("--decoder-seqs", type=int, default=128)
    ap.add_argument("--decoder-seq-len", type=int, default=2048)
    ap.add_argument("--gptaq", action="store_true", help="time the asymmetric-calibration variant instead")
    ap.add_argument("--lora", action="store_true", help="time GPTQ with the low-rank correction instead")
    ap.add_argument("--rank", type=int, default=64)
    ap.add_argument("--lora-iters", type=int, default=10)
    ap.add_argument("--levels", type=int, default=4)
    ap.add_argument("--group-size", type=int, default=64)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the quantizer's "
              "multi-GPU sharding is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import post_weight_quantization_11_amd as g
    from post_weight_quantization_11_amd import _lib

    lib = g.load()
    if args.gemv:
        bench_gemv(args)
        return
    if args.decoder:
        bench_decoder(args)
        return
    if args.gptaq:
        bench_gptaq(args)
        return
    if args.lora:
        bench_lora(args)
        return
    cfg = wl.WORKLOADS[args.config]
    layer = cfg.layers[0]
    m, n, N = layer.m, layer.n, cfg.tokens
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    L = wl.workload_layer(args.config, 0)
    X = L.x_all()
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s: W {m}x{n} {cfg.dtype}, X {N}x{n}")
    Wd = to_device(L.W)
    Xd = to_device(X)
    torch.cuda.synchronize()

    # Outputs and workspaces allocated once, outside the timed region.
    dev = Wd.device
    H = torch.empty((n, n), dtype=torch.float32, device=dev)
    U = torch.empty((n, n), dtype=torch.float32, device=dev)
    perm = torch.empty((n,), dtype=torch.int32, device=dev)
    G = 1 if cfg.group_size == 0 else -(-n // cfg.group_size)
    out = dict(codes=torch.empty((m, n), dtype=torch.uint8, device=dev),
               scales=torch.empty((m, G), dtype=torch.float32, device=dev),
               zeros=torch.empty((m, G), dtype=torch.uint8, device=dev),
               row_loss=torch.empty((m,), dtype=torch.float32, device=dev))
    bits = bits_of(cfg.levels)
    packed = torch.empty((m, g.packed_words(n, bits)), dtype=torch.int32, device=dev)
    gidx = torch.empty((n,), dtype=torch.int32, device=dev)
    xdt = _lib._dtype_code(Xd)
    ws_h = torch.empty(max(1, lib.gptq_hessian_ws_bytes(n, N, xdt)), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(max(1, lib.gptq_prepare_ws_bytes(n)), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(max(1, lib.gptq_quantize_ws_bytes(m, n, _lib._dtype_code(Wd), int(cfg.act_order),
                                                         cfg.block_size)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        g.gptq_hessian_accumulate(H, Xd, 2.0, True, ws=ws_h)
        if ev:
            ev[1].record(stream)
        g.gptq_prepare_hinv(H, cfg.damp_rel, cfg.act_order, U=U, perm=perm, ws=ws_p)
        if ev:
            ev[2].record(stream)
        g.gptq_quantize_layer(Wd, U, perm if cfg.act_order else None, cfg.levels, cfg.group_size,
                              cfg.block_size, out=out, ws=ws_q)
        if ev:
            ev[3].record(stream)
        g.gptq_pack(out["codes"], perm if cfg.act_order else None, bits, cfg.group_size,
                    packed=packed, g_idx=gidx)
        if ev:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_names = ["hessian", "prepare", "quantize", "pack"]
    st_ms = {k: float(np.mean([events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]))
             for i, k in enumerate(stage_names)}
    ms_per_step = wall * 1e3 / args.steps

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # Sanity of the result (not a parity check; the tests do that).
    codes_ok = bool(int(out["codes"].max().item()) <= cfg.levels - 1)
    finite = bool(torch.isfinite(out["scales"]).all().item() and torch.isfinite(out["row_loss"]).all().item())

    flops_h = float(n) * (n + 1) * N
    flops_p = 2.0 / 3.0 * float(n) ** 3
    flops_u = float(m) * n * (n - cfg.block_size)
    in_bytes = {"bf16": 2, "f16": 2, "f32": 4}[cfg.dtype]
    bytes_sweep = float(m) * n * (in_bytes + 4 + 1) + m * G * 5 + n * cfg.block_size * 4
    bytes_pack = float(m) * n * (1 + bits / 8) + 8 * n
    stages = {
        "hessian": {"ms": st_ms["hessian"], "tflops": flops_h / st_ms["hessian"] / 1e9,
                    "frac_peak": flops_h / st_ms["hessian"] / 1e9 / PEAK_BF16_TFLOPS, "peak": "bf16 MFMA 2500 TF"},
        "prepare": {"ms": st_ms["prepare"], "tflops": flops_p / st_ms["prepare"] / 1e9,
                    "frac_peak": flops_p / st_ms["prepare"] / 1e9 / PEAK_F64_TFLOPS, "peak": "f64 78.6 TF"},
        "quantize": {"ms": st_ms["quantize"], "update_tflops": flops_u / st_ms["quantize"] / 1e9,
                     "update_frac_f32_peak": flops_u / st_ms["quantize"] / 1e9 / PEAK_F32_TFLOPS,
                     "sweep_GBps": bytes_sweep / st_ms["quantize"] / 1e6},
        "pack": {"ms": st_ms["pack"], "GBps": bytes_pack / st_ms["pack"] / 1e6,
                 "frac_hbm": bytes_pack / st_ms["pack"] / 1e6 / PEAK_HBM_GBS},
    }
    ms_layer = sum(st_ms.values())
    rec = {
        "metric": METRIC,
        "value": n / (ms_per_step / 1e3),
        "unit": "columns/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "m": m, "n": n, "tokens": N, "x_dtype": cfg.dtype,
                   "levels": cfg.levels, "group_size": cfg.group_size, "block_size": cfg.block_size,
                   "damp_rel": cfg.damp_rel, "act_order": cfg.act_order, "parallelism": "1 GPU"},
        "ms_per_layer_events": ms_layer,
        "weights_per_s": m * n / (ms_per_step / 1e3),
        "stages": stages,
        "roofline": {
            "kernel": "gptq_hessian_accumulate (syrk16 MFMA + split reduce), HIP events around the call",
            "bound": "mfma",
            "achieved": flops_h / st_ms["hessian"] / 1e9,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": flops_h / st_ms["hessian"] / 1e9 / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(args.config),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, copy-calibrated)",
            "algorithmic": f"n(n+1)N = {flops_h:.4g} flop per launch",
        },
        "sanity": {"codes_in_range": codes_ok, "finite": finite},
    }
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(L, X, cfg, n, m, N)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
