// Stage 1: H += alpha * X^T X (GPTQ knowledge note, "How It Works": the
// Hessian of the layer-output loss is H = 2 X X^T over the recorded inputs).
//
// X is tokens x n (token-major, features contiguous).  H is symmetric, so only
// upper 256 x 256 tiles (I <= J) are computed, on MFMA:
//   16-bit X: v_mfma_f32_32x32x16_{bf16,f16} (products exact in float32)
//   32-bit X: v_mfma_f32_32x32x2_f32
// A workgroup (4 waves, 2 x 2 of 128 x 128) owns one tile and one token
// range ("split").  Per stage it loads a 64-token slab of both 256-feature
// bands; each thread loads an 8 x 8 (token x feature) block with 16-byte
// loads, transposes it in registers and stores it feature-major in LDS, so
// every MFMA operand is one 16-byte LDS read.  The LDS pitch (144 B) keeps
// both the transposed stores and the fragment reads free of bank conflicts.
// LDS is double buffered and the next slab is prefetched into registers
// while the current one is multiplied.
//
// Accuracy: one float32 MFMA accumulator covers at most 32768 tokens (a
// "split"); each split writes its tile to the workspace and the reduce
// kernel sums the splits in float64, scales by alpha, adds the old H and
// mirrors the upper triangle.
#include "common.h"

namespace gptq {
namespace {

constexpr int kTile = 256;
constexpr int kThreads = 256;
constexpr int kTileElems = kTile * kTile;

// 16-bit path
constexpr int kKt16 = 64;              // tokens per stage
constexpr int kPitch16 = kKt16 + 8;    // 16-bit elements per LDS row (144 B)

// 32-bit path
constexpr int kKt32 = 16;
constexpr int kPitch32 = kKt32 + 1;

// Longest token range summed in one float32 MFMA accumulator; longer inputs
// are split and the splits are summed in float64.
constexpr int64_t kMaxSplitTokens = 32768;

__device__ inline void tile_coords(int t, int nb, int& I, int& J) {
  int i = 0;
  while (t >= nb - i) {
    t -= nb - i;
    ++i;
  }
  I = i;
  J = i + t;
}

template <int DT> struct Mfma16;
template <> struct Mfma16<GPTQ_BF16> {
  static __device__ inline floatx16 run(u32x4 a, u32x4 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma16<GPTQ_F16> {
  static __device__ inline floatx16 run(u32x4 a, u32x4 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                  __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
  }
};

// Partial-buffer layout of one tile: for wave w, row block rb, column block
// cb (32 x 32 MFMA blocks), register quad q and lane l, 4 consecutive floats
// at ((((w*4 + rb)*4 + cb)*4 + q)*64 + l)*4.  Register r of a 32x32 MFMA
// accumulator holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ inline void store_acc(const floatx16 (&acc)[4][4], float* __restrict__ dst, int wave,
                                 int lane) {
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        floatx4* p = reinterpret_cast<floatx4*>(dst + ((((wave * 4 + rb) * 4 + cb) * 4 + q) * 64 + lane) * 4);
        *p = floatx4{acc[rb][cb][4 * q], acc[rb][cb][4 * q + 1], acc[rb][cb][4 * q + 2],
                     acc[rb][cb][4 * q + 3]};
      }
}

template <int DT>
__global__ __launch_bounds__(kThreads, 1) void syrk16_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int n, int64_t tokens, int nb, int ntiles,
    int nsplit, int64_t tok_per_split, float* __restrict__ partial, int64_t launched, int vec_ok) {
  const int64_t item = xcd_contiguous(blockIdx.x, launched);
  if (item >= (int64_t)ntiles * nsplit) return;
  const int split = (int)(item / ntiles);
  const int tile = (int)(item % ntiles);
  int I, J;
  tile_coords(tile, nb, I, J);
  const int64_t t_begin = (int64_t)split * tok_per_split;
  const int64_t t_end = min(tokens, t_begin + tok_per_split);

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kTile][kPitch16];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tg = lane & 7;                  // loader: token group of 8
  const int fc = wave * 8 + (lane >> 3);    // loader: feature chunk of 8 (0..31)
  const int wr = wave >> 1, wc = wave & 1;  // compute quadrant

  u32x4 pre[2][8];

  auto gload = [&](int64_t t0) {
#pragma unroll
    for (int band = 0; band < 2; ++band) {
      const int f0 = (band == 0 ? I : J) * kTile + fc * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = t0 + tg * 8 + i;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (t < t_end && f0 < n) {
          const uint16_t* p = X + t * ldx + f0;
          if (vec_ok && f0 + 8 <= n) {
            v = *reinterpret_cast<const u32x4*>(p);
          } else {
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (f0 + e < n) ? (uint32_t)p[e] : 0u;
            v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
          }
        }
        pre[band][i] = v;
      }
    }
  };

  auto lstore = [&](int buf) {
#pragma unroll
    for (int band = 0; band < 2; ++band) {
#pragma unroll
      for (int f2 = 0; f2 < 4; ++f2) {
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t y = pre[band][2 * e][f2];      // token 2e: features 2f2 (lo) and 2f2+1 (hi)
          const uint32_t x = pre[band][2 * e + 1][f2];  // token 2e+1
          lo[e] = (y & 0xFFFFu) | (x << 16);
          hi[e] = (y >> 16) | (x & 0xFFFF0000u);
        }
        *reinterpret_cast<u32x4*>(&lds[buf][band][fc * 8 + 2 * f2][tg * 8]) = lo;
        *reinterpret_cast<u32x4*>(&lds[buf][band][fc * 8 + 2 * f2 + 1][tg * 8]) = hi;
      }
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = floatx16{};

  float* dst = partial + ((int64_t)split * ntiles + tile) * (int64_t)kTileElems;
  const int64_t nstages = (t_end - t_begin + kKt16 - 1) / kKt16;
  const int arow = wr * 128 + (lane & 31);
  const int bcol = wc * 128 + (lane & 31);
  const int koff = (lane >> 5) * 8;

  gload(t_begin);
  lstore(0);
  __syncthreads();
  for (int64_t s = 0; s < nstages; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < nstages) gload(t_begin + (s + 1) * kKt16);
#pragma unroll
    for (int kk = 0; kk < kKt16 / 16; ++kk) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        a[rb] = *reinterpret_cast<const u32x4*>(&lds[buf][0][arow + rb * 32][kk * 16 + koff]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        b[cb] = *reinterpret_cast<const u32x4*>(&lds[buf][1][bcol + cb * 32][kk * 16 + koff]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = Mfma16<DT>::run(a[rb], b[cb], acc[rb][cb]);
    }
    if (s + 1 < nstages) lstore(buf ^ 1);
    __syncthreads();
  }
  store_acc(acc, dst, wave, lane);
}

__global__ __launch_bounds__(kThreads, 1) void syrk32_kernel(
    const float* __restrict__ X, int64_t ldx, int n, int64_t tokens, int nb, int ntiles, int nsplit,
    int64_t tok_per_split, float* __restrict__ partial, int64_t launched) {
  const int64_t item = xcd_contiguous(blockIdx.x, launched);
  if (item >= (int64_t)ntiles * nsplit) return;
  const int split = (int)(item / ntiles);
  const int tile = (int)(item % ntiles);
  int I, J;
  tile_coords(tile, nb, I, J);
  const int64_t t_begin = (int64_t)split * tok_per_split;
  const int64_t t_end = min(tokens, t_begin + tok_per_split);

  __shared__ float lds[2][kTile][kPitch32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1;

  floatx16 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = floatx16{};

  float* dst = partial + ((int64_t)split * ntiles + tile) * (int64_t)kTileElems;
  const int64_t nstages = (t_end - t_begin + kKt32 - 1) / kKt32;
  for (int64_t s = 0; s < nstages; ++s) {
    const int64_t t0 = t_begin + s * kKt32;
    // Load both bands: 2 x 256 features x 16 tokens, one element per iteration.
    for (int idx = tid; idx < 2 * kTile * kKt32; idx += kThreads) {
      const int band = idx / (kTile * kKt32);
      const int rem = idx % (kTile * kKt32);
      const int tk = rem / kTile, f = rem % kTile;
      const int gf = (band == 0 ? I : J) * kTile + f;
      const int64_t t = t0 + tk;
      lds[band][f][tk] = (t < t_end && gf < n) ? X[t * ldx + gf] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k2 = 0; k2 < kKt32 / 2; ++k2) {
      float a[4], b[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) a[rb] = lds[0][wr * 128 + rb * 32 + (lane & 31)][k2 * 2 + (lane >> 5)];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) b[cb] = lds[1][wc * 128 + cb * 32 + (lane & 31)][k2 * 2 + (lane >> 5)];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
    }
    __syncthreads();
  }
  store_acc(acc, dst, wave, lane);
}

// One workgroup per 32 x 32 block of an upper tile: sums the splits in
// float64, applies alpha (and the old H unless reset), writes the block and
// its mirror image.
__global__ __launch_bounds__(kThreads) void syrk_reduce_kernel(
    float* __restrict__ H, int n, int nb, int ntiles, int nsplit, const float* __restrict__ partial,
    double alpha, int reset) {
  const int blk = blockIdx.x & 63;
  const int tile = blockIdx.x >> 6;
  int I, J;
  tile_coords(tile, nb, I, J);
  const int wave = blk >> 4, rb = (blk >> 2) & 3, cb = blk & 3;
  const int gr0 = I * kTile + (wave >> 1) * 128 + rb * 32;
  const int gc0 = J * kTile + (wave & 1) * 128 + cb * 32;
  if (gr0 >= n || gc0 >= n || gr0 >= gc0 + 32) return;  // outside, or strictly below the diagonal

  __shared__ double t[32][33];
  const int tid = threadIdx.x, q = tid >> 6, lane = tid & 63;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int sp = 0; sp < nsplit; ++sp) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(
        partial + ((int64_t)sp * ntiles + tile) * (int64_t)kTileElems + (((blk * 4 + q) * 64 + lane) * 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += (double)v[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) t[8 * q + 4 * (lane >> 5) + e][lane & 31] = alpha * s[e];
  __syncthreads();
  {
    const int i = tid >> 3, c0 = (tid & 7) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + e;
      const int gr = gr0 + i, gc = gc0 + c;
      if (gr < n && gc < n && gr <= gc) {
        double v = t[i][c];
        if (!reset) v += (double)H[(int64_t)gr * n + gc];
        H[(int64_t)gr * n + gc] = (float)v;
        t[i][c] = v;
      }
    }
  }
  __syncthreads();
  {
    const int j = tid >> 3, i0 = (tid & 7) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e;
      const int gr = gr0 + i, gc = gc0 + j;
      if (gr < n && gc < n && gr < gc) H[(int64_t)gc * n + gr] = (float)t[i][j];
    }
  }
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

struct SyrkPlan {
  int nb = 0, ntiles = 0, nsplit = 0;
  int64_t tok_per_split = 0;
  int64_t launched = 0;
};

// Chooses the number of token splits (at least tokens / kMaxSplitTokens) so
// that tiles x splits fills the 256 CUs in whole rounds: minimises rounds x
// tokens-per-split, preferring fewer splits (less reduction traffic) within
// 2% of the best.
SyrkPlan plan_syrk(int64_t n, int64_t tokens, int dtype) {
  SyrkPlan p;
  p.nb = (int)ceil_div(n, kTile);
  p.ntiles = p.nb * (p.nb + 1) / 2;
  const int64_t kt = dtype == GPTQ_F32 ? kKt32 : kKt16;
  const int64_t cus = 256;
  double best = 1e300;
  struct Cand { int s; int64_t tps; double cost; };
  Cand cands[65];
  int nc = 0;
  const int s_min = (int)ceil_div(tokens, kMaxSplitTokens);
  for (int s = s_min; s <= s_min + 64; ++s) {
    const int64_t tps = round_up(ceil_div(tokens, s), kt);
    if (s > s_min && tps * (s - 1) >= tokens) break;  // a split would be empty
    if (s > s_min && tps < 4 * kt) break;
    const double rounds = (double)ceil_div((int64_t)p.ntiles * s, cus);
    const double cost = rounds * (double)tps;
    cands[nc++] = {s, tps, cost};
    if (cost < best) best = cost;
  }
  for (int i = 0; i < nc; ++i)
    if (cands[i].cost <= best * 1.02) {
      p.nsplit = cands[i].s;
      p.tok_per_split = cands[i].tps;
      break;
    }
  p.launched = round_up((int64_t)p.ntiles * p.nsplit, kXcds);
  return p;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_hessian_ws_bytes(int64_t n, int64_t tokens, int x_dtype) {
  if (n <= 0 || tokens <= 0 || !valid_dtype(x_dtype)) return 0;
  const SyrkPlan p = plan_syrk(n, tokens, x_dtype);
  return (size_t)p.nsplit * (size_t)p.ntiles * (size_t)kTileElems * sizeof(float);
}

extern "C" gptq_status gptq_hessian_accumulate(float* H, int64_t n, const void* X, int x_dtype,
                                               int64_t tokens, int64_t ldx, float alpha, int reset,
                                               void* ws, size_t ws_bytes, void* stream) {
  if (n < 0 || tokens < 0 || !valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (n > (int64_t)1 << 16) return GPTQ_ERR_UNSUPPORTED;
  if (n == 0) return GPTQ_OK;
  if (H == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (tokens > 0 && (X == nullptr || ldx < n)) return GPTQ_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (tokens == 0) {
    if (reset) {
      fill_zero_kernel<<<1024, 256, 0, st>>>(H, n * n);
      GPTQ_TRY_LAUNCH();
    }
    return GPTQ_OK;
  }
  const SyrkPlan p = plan_syrk(n, tokens, x_dtype);
  const size_t need = (size_t)p.nsplit * (size_t)p.ntiles * (size_t)kTileElems * sizeof(float);
  if (ws == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  float* partial = static_cast<float*>(ws);
  if (x_dtype == GPTQ_F32) {
    syrk32_kernel<<<(unsigned)p.launched, kThreads, 0, st>>>(
        static_cast<const float*>(X), ldx, (int)n, tokens, p.nb, p.ntiles, p.nsplit, p.tok_per_split,
        partial, p.launched);
  } else {
    const int vec_ok = (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    if (x_dtype == GPTQ_BF16)
      syrk16_kernel<GPTQ_BF16><<<(unsigned)p.launched, kThreads, 0, st>>>(
          static_cast<const uint16_t*>(X), ldx, (int)n, tokens, p.nb, p.ntiles, p.nsplit,
          p.tok_per_split, partial, p.launched, vec_ok);
    else
      syrk16_kernel<GPTQ_F16><<<(unsigned)p.launched, kThreads, 0, st>>>(
          static_cast<const uint16_t*>(X), ldx, (int)n, tokens, p.nb, p.ntiles, p.nsplit,
          p.tok_per_split, partial, p.launched, vec_ok);
  }
  GPTQ_TRY_LAUNCH();
  syrk_reduce_kernel<<<(unsigned)p.ntiles * 64u, kThreads, 0, st>>>(H, (int)n, p.nb, p.ntiles, p.nsplit,
                                                                   partial, (double)alpha, reset);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}
