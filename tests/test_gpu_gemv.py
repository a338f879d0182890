"""Parity of the packed-weight matrix-vector product (gptq_dequant_gemv,
through the C ABI) with the oracle's dequant_matmul.

Inputs are seeded codes, scales and zeros packed by the oracle; X is float16
on both sides.  The bar is the float32 rounding bound of the kernel's
arithmetic: every segment of 32 columns is summed as s (sum c x - z sum x) or,
per code, s (c - z) x, so |Y - Y_oracle| <= (n/32 + 80) 2^-23 M with
M = sum_k s (c + z) |x| (oracle.dequant_matmul_bound).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g(gpu_lib):
    import post_weight_quantization_11_amd as g
    return g


def _layer(m, n, bits, group, act, seed, ld_extra=0):
    """Seeded packed layer: codes, per-group scales/zeros, g_idx as gptq_quantize_layer gives it."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 31])))
    maxq = (1 << bits) - 1
    codes = rng.integers(0, maxq + 1, size=(m, n), dtype=np.int64)
    G = 1 if group == 0 else -(-n // group)
    scales = (rng.uniform(0.5, 2.0, size=(m, G)) * 1e-2).astype(np.float32)
    zeros = rng.integers(0, maxq + 1, size=(m, G)).astype(np.uint8)
    perm = rng.permutation(n) if act else np.arange(n)
    g_idx = oracle.group_index(perm, group)
    words = oracle.pack_codes(codes, bits)
    packed = np.zeros((m, words.shape[1] + ld_extra), dtype=np.uint32)
    packed[:, :words.shape[1]] = words
    return dict(packed=packed, nw=words.shape[1], scales=scales, zeros=zeros, g_idx=g_idx, G=G)


def _x(batch, n, seed, ldx=None):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 32])))
    x = rng.standard_normal((batch, n)).astype(np.float16)
    if ldx is None:
        return x, x
    buf = np.zeros((batch, ldx), dtype=np.float16)
    buf[:, :n] = x
    return x, buf


def _run(g, L, X16, Xbuf, n, bits, group, pass_gidx):
    import torch
    packed = torch.from_numpy(L["packed"].view(np.int32)).cuda()
    xd = torch.from_numpy(Xbuf).cuda()[:, :n] if Xbuf.shape[1] != n else torch.from_numpy(Xbuf).cuda()
    Y = g.gptq_dequant_gemv(packed, dev(L["scales"]), dev(L["zeros"], "u8"), xd, n, bits,
                            group_size=group, g_idx=dev(L["g_idx"], "i32") if pass_gidx else None)
    torch.cuda.synchronize()
    return host(Y).astype(np.float64)


def _check(Y, L, X16, n, bits):
    words = L["packed"][:, :L["nw"]]
    Yo = oracle.dequant_matmul(words, n, bits, L["scales"], L["zeros"], L["g_idx"], X16.astype(np.float64))
    M = oracle.dequant_matmul_bound(words, n, bits, L["scales"], L["zeros"], L["g_idx"], X16.astype(np.float64))
    tol = (n / 32 + 80) * 2.0 ** -23 * M
    err = np.abs(Y - Yo)
    log(f"  max |err| / tol = {float(np.max(err / np.maximum(tol, 1e-300))):.3e}")
    assert np.all(err <= tol)


CASES = [
    # m, n, bits, group, act, pass g_idx, batch
    (70, 1000, 4, 0, False, False, 1),      # per-row grid, ragged n and m
    (64, 4096, 4, 128, False, False, 1),    # contiguous groups
    (96, 1024, 3, 128, True, True, 3),      # act-order groups through g_idx
    (33, 500, 2, 64, False, False, 8),      # 2-bit g64, full batch
    (48, 777, 3, 0, False, False, 2),       # 3-bit per-row, words straddle
    (40, 640, 4, 128, False, True, 4),      # contiguous groups passed as g_idx
    (20, 320, 2, 16, False, False, 5),      # groups narrower than a segment
    (1, 33, 4, 0, False, False, 1),         # one row, one column past a segment
    (77, 1000, 4, 128, False, False, 3),    # batch >= 3, contiguous groups: matrix-core kernel
    (50, 640, 2, 0, False, False, 8),       # per-row, full batch: matrix-core kernel
    (3000, 1280, 4, 0, False, False, 1),    # decode kernel with X in LDS: lanes past the last segment
    (200, 8192, 2, 64, False, False, 1),    # decode kernel with X in LDS: 2-bit, groups of 64
    (48, 520, 4, 8, False, False, 1),       # groups of 8 columns
    (30, 264, 3, 2, True, True, 4),         # act-order groups of 2 through g_idx
    (25, 300, 2, 1, False, False, 6),       # one column per group
]


@pytest.mark.parametrize("m,n,bits,group,act,pass_gidx,batch", CASES)
def test_dequant_gemv_parity(g, m, n, bits, group, act, pass_gidx, batch):
    log(f"dequant_gemv m={m} n={n} bits={bits} group={group} act={act} g_idx={pass_gidx} batch={batch}")
    L = _layer(m, n, bits, group, act, seed=m * 7 + n + bits)
    X16, Xbuf = _x(batch, n, seed=n + batch)
    Y = _run(g, L, X16, Xbuf, n, bits, group, pass_gidx)
    _check(Y, L, X16, n, bits)


@pytest.mark.parametrize("m,n,bits,group", [(64, 4096, 4, 128), (3000, 1280, 4, 0), (200, 8192, 2, 64),
                                           (96, 12288, 4, 0)])
def test_dequant_gemv_decode_kernel_matches_row_group_kernel(g, m, n, bits, group):
    # One or two rows of X with aligned rows (n a multiple of 32, segments
    # sharing a group) run on the decode kernel that keeps X in LDS; the same
    # two rows with a padded, unaligned row stride of X run on the row-group
    # kernel.  Both sum each lane's segments in the same order and reduce over
    # the wave the same way, so the results must agree bit for bit.
    log(f"dequant_gemv decode kernel vs row-group kernel m={m} n={n} bits={bits} group={group}")
    L = _layer(m, n, bits, group, False, seed=m + n + 3 * bits)
    X16, Xbuf = _x(2, n, seed=n + 11)
    _, Xpad = _x(2, n, seed=n + 11, ldx=n + 5)
    Y1 = _run(g, L, X16[:1], Xbuf[:1], n, bits, group, False)
    Y2 = _run(g, L, X16, Xbuf, n, bits, group, False)
    Yref = _run(g, L, X16, Xpad, n, bits, group, False)
    _check(Y2, L, X16, n, bits)
    assert np.array_equal(Y1[0], Yref[0])
    assert np.array_equal(Y2, Yref)


# Decode batches of 3 to 16 rows of X on layers of at least 1024 tiles of 16
# rows, or 768 with more than eight rows of X (per-row grids or contiguous
# groups of a multiple of 128 columns, 2- or 4-bit, n a multiple of 32,
# aligned rows) run on the streaming kernel that stages X (and, for groups,
# the rows' scales and zeros) in LDS panels of 512 columns; the cases cover
# one, two and three tiles per wave, a ragged last tile, panels of fewer than
# four chunks, an odd panel count, every staged X width, groups of one, two
# and three chunks and a partial last group.
STREAM_CASES = [
    # m, n, bits, group, batch, entry
    (16390, 1024, 4, 0, 3, "gemv"),      # one tile per wave, ragged last tile, two panels, 4 staged rows
    (32768, 1376, 4, 0, 8, "gemv"),      # two tiles per wave, 43 segments: partial last chunk, three panels
    (24576, 2080, 2, 0, 16, "gemv"),     # 2-bit, 16 rows of X, five panels
    (49152, 640, 4, 0, 12, "gemv"),      # three tiles per wave, 16 staged rows, 12 used
    (20000, 384, 4, 0, 2, "gemm"),       # one panel of three chunks through the matrix-core entry at batch 2
    (16384, 512, 2, 0, 21, "gemm"),      # batch past one 16-row pass: 16 + 5
    (12288, 1056, 4, 0, 12, "gemv"),     # 768 tiles: taken for more than eight rows of X only
    (16390, 1024, 4, 128, 3, "gemv"),    # groups of one chunk, one tile per wave
    (32768, 1376, 4, 256, 8, "gemv"),    # groups of two chunks, partial last group, two tiles per wave
    (49152, 640, 4, 128, 12, "gemv"),    # groups, three tiles per wave
    (24576, 2080, 2, 384, 16, "gemv"),   # 2-bit, groups of three chunks, partial last group
    (12288, 1056, 4, 128, 9, "gemv"),    # groups on a 768-tile layer
]


@pytest.mark.parametrize("m,n,bits,group,batch,entry", STREAM_CASES)
def test_dequant_streaming_kernel(g, m, n, bits, group, batch, entry):
    log(f"dequant streaming kernel m={m} n={n} bits={bits} group={group} batch={batch} entry={entry}")
    L = _layer(m, n, bits, group, False, seed=m + n + batch + group)
    X16, Xbuf = _x(batch, n, seed=5 * n + batch)
    Y = _run(g, L, X16, Xbuf, n, bits, group, False) if entry == "gemv" else _run_gemm(g, L, Xbuf, n, bits, group)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([m, n, 41])))
    rows = np.unique(np.concatenate([rng.choice(m, size=256, replace=False), [0, 15, 16, m - 16, m - 1]]))
    words = L["packed"][rows, :L["nw"]]
    Yo = oracle.dequant_matmul(words, n, bits, L["scales"][rows], L["zeros"][rows], L["g_idx"], X16.astype(np.float64))
    M = oracle.dequant_matmul_bound(words, n, bits, L["scales"][rows], L["zeros"][rows], L["g_idx"],
                                    X16.astype(np.float64))
    tol = (n / 32 + 80) * 2.0 ** -23 * M
    err = np.abs(Y[:, rows] - Yo)
    log(f"  max |err| / tol = {float(np.max(err / np.maximum(tol, 1e-300))):.3e}")
    assert np.all(err <= tol)
    assert np.all(np.isfinite(Y))


def test_dequant_gemv_padded_strides(g):
    # ld_packed and ldx above the minimum (and not multiples of the vector
    # width): the unaligned path.
    m, n, bits, group = 50, 1000, 4, 64
    log("dequant_gemv padded strides")
    L = _layer(m, n, bits, group, False, seed=5, ld_extra=3)
    X16, Xbuf = _x(2, n, seed=6, ldx=n + 5)
    Y = _run(g, L, X16, Xbuf, n, bits, group, False)
    _check(Y, L, X16, n, bits)


def test_dequant_gemv_edges(g):
    import torch
    import post_weight_quantization_11_amd._lib as Lb
    log("dequant_gemv edges")
    L = _layer(8, 64, 4, 0, False, seed=1)
    packed = torch.from_numpy(L["packed"].view(np.int32)).cuda()
    s, z = dev(L["scales"]), dev(L["zeros"], "u8")
    # batch 0 is an error for the decode call
    with pytest.raises(Lb.GptqError) as ei:
        g.gptq_dequant_gemv(packed, s, z, torch.zeros((0, 64), dtype=torch.float16, device="cuda"), 64, 4)
    assert ei.value.status == Lb.GPTQ_ERR_INVALID_ARG
    # unsupported bit width
    with pytest.raises(Lb.GptqError) as ei:
        g.gptq_dequant_gemv(packed, s, z, torch.zeros((1, 64), dtype=torch.float16, device="cuda"), 64, 5)
    assert ei.value.status == Lb.GPTQ_ERR_INVALID_ARG
    # too few groups for the group size
    with pytest.raises(Lb.GptqError) as ei:
        g.gptq_dequant_gemv(packed, s, z, torch.zeros((1, 64), dtype=torch.float16, device="cuda"), 64, 4,
                            group_size=32)
    assert ei.value.status == Lb.GPTQ_ERR_INVALID_ARG
    # n = 0: Y is all zero
    Y = g.gptq_dequant_gemv(packed[:, :0], s, z, torch.zeros((2, 0), dtype=torch.float16, device="cuda"), 0, 4,
                            Y=torch.full((2, 8), 7.0, device="cuda"))
    torch.cuda.synchronize()
    assert np.all(host(Y) == 0)


@pytest.mark.parametrize("batch,group", [(1, 0), (2, 0), (4, 0), (16, 0), (4, 128), (16, 128)])
def test_dequant_gemv_full_size_layer(g, batch, group):
    # The 175B-class fc1 layer (49152 x 12288, 4-bit) at the batches the
    # decode measurements time (1 and 16 in the bench line's next rows, 4 in
    # its profile) and with groups of 128; sampled rows against the oracle.
    import torch
    m, n, bits = 49152, 12288, 4
    log(f"dequant_gemv full size 49152 x 12288 batch {batch} group {group}")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([11, 33, batch, group])))
    nw = oracle.packed_words_per_row(n, bits)
    G = 1 if group == 0 else n // group
    words = rng.integers(0, 1 << 32, size=(m, nw), dtype=np.uint64).astype(np.uint32)
    scales = (rng.uniform(0.5, 2.0, size=(m, G)) * 1e-2).astype(np.float32)
    zeros = rng.integers(0, 16, size=(m, G)).astype(np.uint8)
    g_idx = (np.arange(n) // group if group else np.zeros(n)).astype(np.int32)
    X16 = rng.standard_normal((batch, n)).astype(np.float16)
    Y = g.gptq_dequant_gemv(torch.from_numpy(words.view(np.int32)).cuda(), dev(scales), dev(zeros, "u8"),
                            torch.from_numpy(X16).cuda(), n, bits, group_size=group)
    torch.cuda.synchronize()
    Yg = host(Y).astype(np.float64)
    rows = np.sort(rng.choice(m, size=64, replace=False))
    rows[0], rows[-1] = 0, m - 1
    Yo = oracle.dequant_matmul(words[rows], n, bits, scales[rows], zeros[rows], g_idx, X16.astype(np.float64))
    M = oracle.dequant_matmul_bound(words[rows], n, bits, scales[rows], zeros[rows], g_idx, X16.astype(np.float64))
    tol = (n / 32 + 80) * 2.0 ** -23 * M
    err = np.abs(Yg[:, rows] - Yo)
    log(f"  max |err| / tol = {float(np.max(err / tol)):.3e}")
    assert np.all(err <= tol)


# ---------------------------------------------------------------------------
# Matrix-core product (gptq_dequant_gemm), any batch.
# ---------------------------------------------------------------------------
def _run_gemm(g, L, Xbuf, n, bits, group, pass_gidx=False):
    import torch
    packed = torch.from_numpy(L["packed"].view(np.int32)).cuda()
    xd = torch.from_numpy(Xbuf).cuda()
    if Xbuf.shape[1] != n:
        xd = xd[:, :n]
    Y = g.gptq_dequant_gemm(packed, dev(L["scales"]), dev(L["zeros"], "u8"), xd, n, bits, group_size=group,
                            g_idx=dev(L["g_idx"], "i32") if pass_gidx else None)
    torch.cuda.synchronize()
    return host(Y).astype(np.float64)


GEMM_CASES = [
    # m, n, bits, group, batch
    (70, 1000, 4, 0, 1),        # ragged m and n, per-row
    (64, 1024, 4, 128, 5),      # contiguous groups, batch inside one tile
    (40, 1000, 3, 128, 16),     # 3-bit, partial last group, full tile
    (33, 500, 2, 256, 17),      # 2-bit, batch past one 16-row chunk
    (64, 768, 4, 128, 40),      # three 16-row chunks, the last one ragged
    (20000, 384, 4, 0, 2),      # many rows (32 rows per wave)
    (96, 640, 4, 128, 100),     # prefill-sized batch (128 x 128 tiles, X staged in LDS)
    (300, 1000, 3, 0, 257),     # prefill, ragged rows, columns and batch, 3-bit
    (130, 512, 2, 256, 130),    # prefill, 2-bit groups of 256
    (60, 520, 4, 8, 24),        # groups of 8 columns (per-code path)
]


# Layouts the matrix-core kernel does not take: act-order groups through
# g_idx and groups narrower than 128 columns, at batches above one VALU pass
# (eight rows of X), through both entry points.
VALU_BATCH_CASES = [
    # m, n, bits, group, act, batch
    (96, 1024, 3, 128, True, 19),      # act-order g128, three passes, the last one ragged
    (70, 640, 4, 64, False, 40),       # g64, five passes
    (33, 500, 2, 16, True, 9),         # act-order groups narrower than a segment
    (257, 4096, 4, 128, True, 64),     # act-order prefill-sized batch
]


@pytest.mark.parametrize("m,n,bits,group,act,batch", VALU_BATCH_CASES)
def test_dequant_products_any_layout_any_batch(g, m, n, bits, group, act, batch):
    import torch
    log(f"dequant product any layout m={m} n={n} bits={bits} group={group} act={act} batch={batch}")
    L = _layer(m, n, bits, group, act, seed=m + n + batch)
    X16, Xbuf = _x(batch, n, seed=3 * n + batch)
    _check(_run_gemm(g, L, Xbuf, n, bits, group, pass_gidx=act), L, X16, n, bits)
    _check(_run(g, L, X16, Xbuf, n, bits, group, pass_gidx=act), L, X16, n, bits)
    if act:
        # the same layer with contiguous groups through g_idx (a permutation
        # that keeps the order) equals the one without g_idx
        Lc = _layer(m, n, bits, group, False, seed=m + n + batch)
        Yg = _run_gemm(g, Lc, Xbuf, n, bits, group, pass_gidx=True)
        _check(Yg, Lc, X16, n, bits)


@pytest.mark.parametrize("m,n,bits,group,batch", GEMM_CASES)
def test_dequant_gemm_parity(g, m, n, bits, group, batch):
    log(f"dequant_gemm m={m} n={n} bits={bits} group={group} batch={batch}")
    L = _layer(m, n, bits, group, False, seed=m + 3 * n + bits)
    X16, Xbuf = _x(batch, n, seed=2 * n + batch)
    Y = _run_gemm(g, L, Xbuf, n, bits, group)
    _check(Y, L, X16, n, bits)


def test_dequant_gemm_padded_strides_and_edges(g):
    import torch
    import post_weight_quantization_11_amd._lib as Lb
    log("dequant_gemm padded strides and edges")
    m, n, bits, group = 50, 1000, 4, 128
    L = _layer(m, n, bits, group, False, seed=8, ld_extra=3)
    X16, Xbuf = _x(3, n, seed=9, ldx=n + 5)
    _check(_run_gemm(g, L, Xbuf, n, bits, group), L, X16, n, bits)
    packed = torch.from_numpy(L["packed"].view(np.int32)).cuda()
    s, z = dev(L["scales"]), dev(L["zeros"], "u8")
    # batch 0 is a no-op
    Y = g.gptq_dequant_gemm(packed, s, z, torch.zeros((0, n), dtype=torch.float16, device="cuda"), n, bits,
                            group_size=group)
    assert tuple(Y.shape) == (0, m)
