// Low-rank correction folded into the GPTQ pass (GPTQ-intrinsic LoRA abstract,
// Daily Papers page).  The weights are approximated as Q + (L R)^T (L n x r,
// R r x m) and judged by ||(W - Q - R^T L^T) X^T||^2.  For a fixed L the best
// R is a least-squares solution, R* = K^T (W - Q)^T with K = H L M^{-1},
// M = L^T H L, H = 2 X^T X, and what remains to minimise over Q is GPTQ's
// objective with the Hessian H_L = H - H L M^{-1} L^T H.  With the Cholesky
// factor M = C C^T and Z = H L C^{-T}:
//   H_L = H - Z Z^T,   K = Z C^{-1}.
// The page's choice L = V_r (top-r right singular vectors of X, i.e. top-r
// eigenvectors of H) is found by subspace iteration, L <- orth(H L), with
// Cholesky-QR as the orthonormalisation; H_L and R* depend on L only through
// its column span.
//
// All arithmetic is float64; H and H_L are float32 (the precision in which
// gptq_hessian_accumulate writes H and gptq_prepare_hinv reads it), R is
// float32.  Matrices of r columns (L, K, Omega and the internal Y, Z) are
// row-major n x r.  The products are small next to the Hessian (n^2 r
// multiply-adds for H L and for H_L, m n r for R*), so they run as plain
// float64 VALU tiles: 64-row output tiles of all r <= 64 columns, 4 x 4 per
// thread, K staged 32 deep through LDS and split over workgroups with a
// fixed-order float64 reduction (results do not depend on timing).
#include "common.h"

namespace gptq {
namespace {

constexpr int kR = GPTQ_LOWRANK_MAX_RANK;  // column tile = the largest rank
constexpr int kThreads = 256;
constexpr int kTP = 64;                    // output rows per workgroup
constexpr int kTK = 32;                    // K per LDS stage
constexpr int kPitch = kTP + 4;            // doubles per LDS row (32-byte aligned rows)
constexpr int kTargetBlocks = 512;

static_assert(kR == 64, "the tile shapes assume a 64-column rank tile");

// A operand of the tall product Out(p, a) = sum_k A(p, k) B(k, a).
enum AMode { kHessianT = 0, kMatT = 1, kDelta = 2 };

struct TallArgs {
  // A
  const void* A;       // kHessianT: float H (n x n, ld); kMatT: double (K x P, ld); kDelta: W (m x n, ld)
  int64_t lda;
  int w_dtype;         // kDelta
  const uint8_t* codes;   // kDelta: m x n, processing order
  const float* scales;    // kDelta: m x G
  const uint8_t* zeros;   // kDelta: m x G
  int64_t G, group;       // kDelta
  const int32_t* perm;    // kDelta: A's column k is W's column perm[k]; B's row k is perm[k]; may be NULL
  // B: K x r float64, row-major (ld r), rows gathered through perm in kDelta
  const double* B;
  int64_t ldb;
  int64_t P, K, r;
  int64_t kchunk;      // K per split (multiple of kTK)
  double* part;        // splits x P x kR
};

template <int DT>
__device__ inline double w_elem(const void* W, int64_t i) {
  return static_cast<double>(load_as_f32<DT>(W, i));
}

template <int MODE, int DT>
__device__ inline void load_a_stage(const TallArgs& a, double (*As)[kPitch], int64_t p0, int64_t k0, int tid) {
  if (MODE == kHessianT || MODE == kMatT) {
    // A(p, k) = Src[k][p]: row k of the source is read contiguously along p.
    const int pp = tid & 63;
#pragma unroll
    for (int it = 0; it < kTK / 4; ++it) {
      const int kk = (tid >> 6) + 4 * it;
      const int64_t p = p0 + pp, k = k0 + kk;
      double v = 0.0;
      if (p < a.P && k < a.K) {
        if (MODE == kHessianT) v = static_cast<double>(static_cast<const float*>(a.A)[k * a.lda + p]);
        else v = static_cast<const double*>(a.A)[k * a.lda + p];
      }
      As[kk][pp] = v;
    }
  } else {
    // A(p, k) = W[p][perm[k]] - s (c - z) for row p, processing column k:
    // exactly the float64 difference of the stored weight and its dequantized
    // value (s is float32 and c - z a small integer, so s (c - z) is exact).
    const int kk = tid & 31;
#pragma unroll
    for (int it = 0; it < kTP / 8; ++it) {
      const int pp = (tid >> 5) + 8 * it;
      const int64_t p = p0 + pp, k = k0 + kk;
      double v = 0.0;
      if (p < a.P && k < a.K) {
        const int64_t col = a.perm ? static_cast<int64_t>(a.perm[k]) : k;
        const int64_t g = a.group ? k / a.group : 0;
        const double s = static_cast<double>(a.scales[p * a.G + g]);
        const double c = static_cast<double>(a.codes[p * a.K + k]);
        const double z = static_cast<double>(a.zeros[p * a.G + g]);
        v = w_elem<DT>(a.A, p * a.lda + col) - s * (c - z);
      }
      As[kk][pp] = v;
    }
  }
}

// part[s][p][a] = sum over split s's K range of A(p, k) B(k, a), for one
// 64-row tile (blockIdx.x) and one split (blockIdx.y).
template <int MODE, int DT>
__global__ __launch_bounds__(kThreads) void tall_product_kernel(TallArgs a) {
  __shared__ __attribute__((aligned(16))) double As[kTK][kPitch];
  __shared__ __attribute__((aligned(16))) double Bs[kTK][kPitch];
  const int tid = threadIdx.x;
  const int tp = tid & 15, ta = tid >> 4;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kTP;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * a.kchunk;
  const int64_t kend = kbeg + a.kchunk < a.K ? kbeg + a.kchunk : a.K;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

  for (int64_t k0 = kbeg; k0 < kend; k0 += kTK) {
    load_a_stage<MODE, DT>(a, As, p0, k0, tid);
    {
      const int col = tid & 63;
#pragma unroll
      for (int it = 0; it < kTK / 4; ++it) {
        const int kk = (tid >> 6) + 4 * it;
        const int64_t k = k0 + kk;
        double v = 0.0;
        if (k < kend && col < a.r) {
          const int64_t row = (MODE == kDelta && a.perm) ? static_cast<int64_t>(a.perm[k]) : k;
          v = a.B[row * a.ldb + col];
        }
        Bs[kk][col] = v;
      }
    }
    // B rows at or past kend are zero, so A's columns there (the next split's) add nothing.
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kTK; ++kk) {
      const doublex4 av = *reinterpret_cast<const doublex4*>(&As[kk][4 * tp]);
      const doublex4 bv = *reinterpret_cast<const doublex4*>(&Bs[kk][4 * ta]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fma(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  double* out = a.part + static_cast<int64_t>(blockIdx.y) * a.P * kR;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t p = p0 + 4 * tp + i;
    if (p < a.P) {
      doublex4 v = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
      *reinterpret_cast<doublex4*>(out + p * kR + 4 * ta) = v;
    }
  }
}

// Sums the splits in split order.  TRANSPOSE_F32: R[a][p] = (float) sum
// (ld ldo); else Out[p][a] = sum (float64, ld ldo).
template <bool TRANSPOSE_F32>
__global__ __launch_bounds__(kThreads) void reduce_splits_kernel(const double* __restrict__ part, int splits,
                                                                 int64_t P, int64_t r, void* __restrict__ out,
                                                                 int64_t ldo) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= P * r) return;
  int64_t p, c;
  if (TRANSPOSE_F32) { c = e / P; p = e % P; }   // consecutive threads write consecutive p of R's row c
  else { p = e / r; c = e % r; }
  double s = 0.0;
  for (int t = 0; t < splits; ++t) s += part[(static_cast<int64_t>(t) * P + p) * kR + c];
  if (TRANSPOSE_F32) static_cast<float*>(out)[c * ldo + p] = static_cast<float>(s);
  else static_cast<double*>(out)[p * ldo + c] = s;
}

// One workgroup: G = sum of the splits of the r x r product (lower triangle
// used), G = C C^T (Cholesky, lower), Cinv = C^{-1} (lower).  C lives in the
// lower triangle of Gs; column c of C^{-1} below its diagonal is built in row c
// of Gs above the diagonal (Gs[c][i] = Cinv[i][c], i > c).  A pivot that is
// not a positive finite number sets *flag to 1; reset clears it first.
__global__ __launch_bounds__(kThreads) void small_cholesky_kernel(const double* __restrict__ part, int splits,
                                                                  int r, double* __restrict__ C,
                                                                  double* __restrict__ Cinv,
                                                                  int32_t* __restrict__ flag, int reset) {
  __shared__ double Gs[kR][kR + 1];
  const int tid = threadIdx.x;
  int bad = 0;  // meaningful in thread 0 only
  for (int e = tid; e < kR * kR; e += kThreads) {
    const int i = e / kR, j = e % kR;
    double s = 0.0;
    if (i < r && j <= i)
      for (int t = 0; t < splits; ++t) s += part[(static_cast<int64_t>(t) * r + i) * kR + j];
    Gs[i][j] = s;
  }
  __syncthreads();
  for (int k = 0; k < r; ++k) {
    if (tid == 0) {
      const double d = Gs[k][k];
      if (!(d > 0.0) || !(d < INFINITY)) {
        bad = 1;
        Gs[k][k] = 1.0;
      } else {
        Gs[k][k] = sqrt(d);
      }
    }
    __syncthreads();
    const double dk = Gs[k][k];
    for (int i = k + 1 + tid; i < r; i += kThreads) Gs[i][k] /= dk;
    __syncthreads();
    const int w = r - k - 1;
    for (int e = tid; e < w * w; e += kThreads) {
      const int i = k + 1 + e / w, j = k + 1 + e % w;
      if (j <= i) Gs[i][j] = __builtin_fma(-Gs[i][k], Gs[j][k], Gs[i][j]);
    }
    __syncthreads();
  }
  // Column c of C^{-1} by forward substitution, one thread per column:
  // X[c][c] = 1 / C[c][c], X[i][c] = -(sum_{k=c}^{i-1} C[i][k] X[k][c]) / C[i][i].
  if (tid < r) {
    const int c = tid;
    const double xcc = 1.0 / Gs[c][c];
    for (int i = c + 1; i < r; ++i) {
      double s = Gs[i][c] * xcc;
      for (int k = c + 1; k < i; ++k) s = __builtin_fma(Gs[i][k], Gs[c][k], s);
      Gs[c][i] = -s / Gs[i][i];
    }
  }
  __syncthreads();
  for (int e = tid; e < kR * kR; e += kThreads) {
    const int i = e / kR, j = e % kR;
    const bool in = i < r && j <= i;
    C[e] = in ? Gs[i][j] : 0.0;
    Cinv[e] = !in ? 0.0 : (i == j ? 1.0 / Gs[i][i] : Gs[j][i]);
  }
  if (tid == 0) {
    const int32_t prev = reset ? 0 : *flag;
    *flag = prev | bad;
  }
}

// Out = Y T for Y n x r, T r x r: TRANS_INV: T = Cinv^T (Y C^{-T});
// else T = Cinv (Z C^{-1}).  16 rows per workgroup.
template <bool TRANS_INV>
__global__ __launch_bounds__(kThreads) void right_multiply_kernel(const double* __restrict__ Y,
                                                                  const double* __restrict__ Cinv, int64_t n,
                                                                  int r, double* __restrict__ Out) {
  __shared__ double Ts[kR][kR + 1];
  __shared__ double Ys[16][kR + 1];
  const int tid = threadIdx.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 16;
  for (int e = tid; e < kR * kR; e += kThreads) {
    const int b = e / kR, c = e % kR;
    Ts[b][c] = TRANS_INV ? Cinv[c * kR + b] : Cinv[b * kR + c];
  }
  for (int e = tid; e < 16 * kR; e += kThreads) {
    const int ii = e / kR, b = e % kR;
    const int64_t i = i0 + ii;
    Ys[ii][b] = (i < n && b < r) ? Y[i * r + b] : 0.0;
  }
  __syncthreads();
  const int c = tid & 63;
  const int ib = (tid >> 6) * 4;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int b = 0; b < r; ++b) {
    const double t = Ts[b][c];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = __builtin_fma(Ys[ib + u][b], t, acc[u]);
  }
  if (c < r) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + ib + u;
      if (i < n) Out[i * r + c] = acc[u];
    }
  }
}

// H_L[i][j] = (float)(H[i][j] - sum_a Z[i][a] Z[j][a]), 64 x 64 tiles.  The
// products and their order are the same for (i, j) and (j, i), so H_L is
// exactly symmetric when H is.
__global__ __launch_bounds__(kThreads) void downdate_kernel(const float* __restrict__ H, int64_t ldh,
                                                            const double* __restrict__ Z, int64_t n, int r,
                                                            float* __restrict__ HL, int64_t ldhl) {
  // Z rows of the tile, transposed ([a][row]); consecutive threads take
  // consecutive rows (conflict-free LDS stores, Z itself is L2-resident).
  __shared__ double Zi[kR][kTP];
  __shared__ double Zj[kR][kTP];
  const int tid = threadIdx.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.y) * kTP, j0 = static_cast<int64_t>(blockIdx.x) * kTP;
  for (int e = tid; e < kR * kTP; e += kThreads) {
    const int rr = e % kTP, a = e / kTP;
    const int64_t i = i0 + rr, j = j0 + rr;
    Zi[a][rr] = (i < n && a < r) ? Z[i * r + a] : 0.0;
    Zj[a][rr] = (j < n && a < r) ? Z[j * r + a] : 0.0;
  }
  __syncthreads();
  const int ti = tid & 15, tj = tid >> 4;
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + 4 * ti + u;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t j = j0 + 4 * tj + v;
      acc[u][v] = (i < n && j < n) ? static_cast<double>(H[i * ldh + j]) : 0.0;
    }
  }
  for (int a = 0; a < r; ++a) {
    double zi[4], zj[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      zi[u] = Zi[a][4 * ti + u];
      zj[u] = Zj[a][4 * tj + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fma(-zi[u], zj[v], acc[u][v]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + 4 * ti + u;
    if (i >= n) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t j = j0 + 4 * tj + v;
      if (j < n) HL[i * ldhl + j] = static_cast<float>(acc[u][v]);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct Split {
  int64_t tiles, splits, kchunk;
};

Split choose_split(int64_t P, int64_t K) {
  Split s;
  s.tiles = ceil_div(P, kTP);
  const int64_t stages = ceil_div(K, kTK);
  // Enough workgroups to cover the chip, at least four K stages per split.
  int64_t want = ceil_div(kTargetBlocks, s.tiles);
  const int64_t cap = std::max<int64_t>(1, stages / 4);
  want = std::max<int64_t>(1, std::min(want, cap));
  s.kchunk = ceil_div(stages, want) * kTK;
  s.splits = ceil_div(K, s.kchunk);
  return s;
}

size_t part_bytes(int64_t P, int64_t K) {
  const Split s = choose_split(P, K);
  return static_cast<size_t>(s.splits) * static_cast<size_t>(P) * kR * sizeof(double);
}

struct Layout {
  size_t off_part, off_y, off_q, off_c, off_cinv, off_flag, total;
};

Layout lowrank_layout(int64_t m, int64_t n, int64_t r) {
  Layout L;
  size_t part = std::max(part_bytes(n, n), part_bytes(r, n));
  if (m > 0) part = std::max(part, part_bytes(m, n));
  const size_t nr = static_cast<size_t>(n) * static_cast<size_t>(r) * sizeof(double);
  L.off_part = 0;
  L.off_y = align256(part);
  L.off_q = align256(L.off_y + nr);
  L.off_c = align256(L.off_q + nr);
  L.off_cinv = align256(L.off_c + kR * kR * sizeof(double));
  L.off_flag = align256(L.off_cinv + kR * kR * sizeof(double));
  L.total = align256(L.off_flag + sizeof(int32_t));
  return L;
}

struct Ctx {
  hipStream_t st;
  double* part;
  double* Y;
  double* Q;
  double* C;
  double* Cinv;
  int32_t* flag;
};

Ctx make_ctx(const Layout& L, void* ws, void* stream) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  Ctx c;
  c.st = static_cast<hipStream_t>(stream);
  c.part = reinterpret_cast<double*>(base + L.off_part);
  c.Y = reinterpret_cast<double*>(base + L.off_y);
  c.Q = reinterpret_cast<double*>(base + L.off_q);
  c.C = reinterpret_cast<double*>(base + L.off_c);
  c.Cinv = reinterpret_cast<double*>(base + L.off_cinv);
  c.flag = reinterpret_cast<int32_t*>(base + L.off_flag);
  return c;
}

template <int MODE, int DT>
gptq_status launch_tall(TallArgs a, const Ctx& c, Split* used) {
  const Split s = choose_split(a.P, a.K);
  a.kchunk = s.kchunk;
  a.part = c.part;
  tall_product_kernel<MODE, DT><<<dim3(static_cast<unsigned>(s.tiles), static_cast<unsigned>(s.splits)),
                                  kThreads, 0, c.st>>>(a);
  GPTQ_TRY_LAUNCH();
  *used = s;
  return GPTQ_OK;
}

// Out (n x r, float64) = H X for X n x r.
gptq_status product_h(const float* H, int64_t ldh, const double* X, int64_t n, int64_t r, double* Out,
                      const Ctx& c) {
  TallArgs a = {};
  a.A = H; a.lda = ldh; a.B = X; a.ldb = r; a.P = n; a.K = n; a.r = r;
  Split s;
  gptq_status rc = launch_tall<kHessianT, GPTQ_F32>(a, c, &s);
  if (rc != GPTQ_OK) return rc;
  reduce_splits_kernel<false><<<static_cast<unsigned>(ceil_div(n * r, kThreads)), kThreads, 0, c.st>>>(
      c.part, static_cast<int>(s.splits), n, r, Out, r);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

// C, Cinv from the Cholesky factor of A^T B (A, B n x r).
gptq_status factor_gram(const double* A, const double* B, int64_t n, int64_t r, const Ctx& c, int reset) {
  TallArgs a = {};
  a.A = A; a.lda = r; a.B = B; a.ldb = r; a.P = r; a.K = n; a.r = r;
  Split s;
  gptq_status rc = launch_tall<kMatT, GPTQ_F32>(a, c, &s);
  if (rc != GPTQ_OK) return rc;
  small_cholesky_kernel<<<1, kThreads, 0, c.st>>>(c.part, static_cast<int>(s.splits), static_cast<int>(r), c.C,
                                                  c.Cinv, c.flag, reset);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

// Out = Y C^{-T} with C from the last factor_gram (orthonormal columns when
// C came from Y^T Y).
gptq_status orthonormalize(const double* Y, int64_t n, int64_t r, double* Out, const Ctx& c, int reset) {
  gptq_status rc = factor_gram(Y, Y, n, r, c, reset);
  if (rc != GPTQ_OK) return rc;
  right_multiply_kernel<true><<<static_cast<unsigned>(ceil_div(n, 16)), kThreads, 0, c.st>>>(
      Y, c.Cinv, n, static_cast<int>(r), Out);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

gptq_status read_flag(const Ctx& c) {
  int32_t h = 0;
  GPTQ_TRY_HIP(hipMemcpyAsync(&h, c.flag, sizeof(int32_t), hipMemcpyDeviceToHost, c.st));
  GPTQ_TRY_HIP(hipStreamSynchronize(c.st));
  return h ? GPTQ_ERR_NOT_PD : GPTQ_OK;
}

bool rank_ok(int64_t n, int64_t r) { return n >= 1 && r >= 1 && r <= kR && r <= n; }

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_lowrank_ws_bytes(int64_t m, int64_t n, int64_t r) {
  if (m < 0 || !rank_ok(n, r)) return 0;
  return lowrank_layout(m, n, r).total;
}

extern "C" gptq_status gptq_lowrank_basis(const float* H, int64_t n, int64_t ldh, int64_t r, const double* Omega,
                                          int iters, double* L, void* ws, size_t ws_bytes, void* stream) {
  if (!H || !Omega || !L || !rank_ok(n, r) || ldh < n || iters < 0) return GPTQ_ERR_INVALID_ARG;
  const Layout lay = lowrank_layout(0, n, r);
  if (!ws || ws_bytes < lay.total) return GPTQ_ERR_WORKSPACE;
  const Ctx c = make_ctx(lay, ws, stream);
  gptq_status rc = orthonormalize(Omega, n, r, L, c, 1);
  for (int it = 0; rc == GPTQ_OK && it < iters; ++it) {
    rc = product_h(H, ldh, L, n, r, c.Y, c);
    if (rc == GPTQ_OK) rc = orthonormalize(c.Y, n, r, L, c, 0);
  }
  // A second Cholesky-QR pass restores orthonormality to float64 accuracy.
  if (rc == GPTQ_OK) rc = orthonormalize(L, n, r, c.Q, c, 0);
  if (rc == GPTQ_OK) {
    GPTQ_TRY_HIP(hipMemcpyAsync(L, c.Q, static_cast<size_t>(n * r) * sizeof(double), hipMemcpyDeviceToDevice,
                                c.st));
    rc = read_flag(c);
  }
  return rc;
}

extern "C" gptq_status gptq_lowrank_hessian(const float* H, int64_t n, int64_t ldh, const double* L, int64_t r,
                                            float* H_L, int64_t ldhl, double* K, void* ws, size_t ws_bytes,
                                            void* stream) {
  if (!H || !L || !H_L || !K || !rank_ok(n, r) || ldh < n || ldhl < n) return GPTQ_ERR_INVALID_ARG;
  if (H_L == H) return GPTQ_ERR_INVALID_ARG;  // tiles read H rows that other tiles write
  const Layout lay = lowrank_layout(0, n, r);
  if (!ws || ws_bytes < lay.total) return GPTQ_ERR_WORKSPACE;
  const Ctx c = make_ctx(lay, ws, stream);
  gptq_status rc = product_h(H, ldh, L, n, r, c.Y, c);                    // Y = H L
  if (rc == GPTQ_OK) rc = factor_gram(L, c.Y, n, r, c, 1);                 // L^T H L = C C^T
  if (rc != GPTQ_OK) return rc;
  right_multiply_kernel<true><<<static_cast<unsigned>(ceil_div(n, 16)), kThreads, 0, c.st>>>(
      c.Y, c.Cinv, n, static_cast<int>(r), c.Q);                          // Z = Y C^{-T}
  GPTQ_TRY_LAUNCH();
  right_multiply_kernel<false><<<static_cast<unsigned>(ceil_div(n, 16)), kThreads, 0, c.st>>>(
      c.Q, c.Cinv, n, static_cast<int>(r), K);                            // K = Z C^{-1}
  GPTQ_TRY_LAUNCH();
  const unsigned t = static_cast<unsigned>(ceil_div(n, kTP));
  downdate_kernel<<<dim3(t, t), kThreads, 0, c.st>>>(H, ldh, c.Q, n, static_cast<int>(r), H_L, ldhl);
  GPTQ_TRY_LAUNCH();
  return read_flag(c);
}

extern "C" gptq_status gptq_lowrank_compensation(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw,
                                                 const uint8_t* codes, const float* scales, const uint8_t* zeros,
                                                 int group_size, const int32_t* perm, const double* K, int64_t r,
                                                 float* R, int64_t ldr, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !codes || !scales || !zeros || !K || !R || !valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (m < 1 || !rank_ok(n, r) || ldw < n || ldr < m || group_size < 0) return GPTQ_ERR_INVALID_ARG;
  const Layout lay = lowrank_layout(m, n, r);
  if (!ws || ws_bytes < lay.total) return GPTQ_ERR_WORKSPACE;
  const Ctx c = make_ctx(lay, ws, stream);
  TallArgs a = {};
  a.A = W; a.lda = ldw; a.w_dtype = w_dtype; a.codes = codes; a.scales = scales; a.zeros = zeros;
  a.group = group_size; a.G = group_size ? ceil_div(n, group_size) : 1; a.perm = perm;
  a.B = K; a.ldb = r; a.P = m; a.K = n; a.r = r;
  Split s;
  gptq_status rc = w_dtype == GPTQ_F32  ? launch_tall<kDelta, GPTQ_F32>(a, c, &s)
                   : w_dtype == GPTQ_F16 ? launch_tall<kDelta, GPTQ_F16>(a, c, &s)
                                         : launch_tall<kDelta, GPTQ_BF16>(a, c, &s);
  if (rc != GPTQ_OK) return rc;
  reduce_splits_kernel<true><<<static_cast<unsigned>(ceil_div(m * r, kThreads)), kThreads, 0, c.st>>>(
      c.part, static_cast<int>(s.splits), m, r, R, ldr);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}
