// Stage 2: damping, act-order and the inverse-Hessian factor U.
// GPTQ knowledge note, "How It Works": a damped Cholesky formulation
// supplies the correction rows.
//
// With J the index-reversal matrix and H_d = H[perm][:, perm] + lambda I:
//   A = J H_d J = L L^T          (ordinary lower Cholesky of the reversed matrix)
//   H_d = R R^T with R = J L J    (R upper)
//   U = R^{-1} = J L^{-1} J       (upper, U^T U = H_d^{-1})
// so one Cholesky and one triangular inverse (2/3 n^3 flops in all) give U
// directly; H_d^{-1} is never formed.  Both run in float64, right-looking
// with 64 x 64 blocks, interleaved in one loop over block columns kb with two
// launches per step:
//   panel(kb)   L[i, kb] = A[i, kb] inv(L_kk)^T                   (MFMA f64)
//               X[kb, j] = inv(L_kk) T[kb, j], j < kb             (MFMA f64)
//   update(kb)  A[i, j] -= L[i, kb] L[j, kb]^T, kb < j <= i       (MFMA f64)
//               T[i, j] -= L[i, kb] X[kb, j], i > kb, j <= kb     (MFMA f64)
//               + the workgroup that updates block (kb+1, kb+1) then factors
//                 it (one wave, no barriers) and inverts it (four waves),
//                 overlapping the rest of the trailing update
// where X = L^{-1} is built in place of T (forward substitution by block
// rows).  Matrices are padded to a multiple of 64 with an identity block.
#include "common.h"

namespace gptq {
namespace {

constexpr int kB = 64;        // Cholesky block
constexpr int kThreads = 256;

__global__ void init_scalars_kernel(int32_t* info) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *info = 0;
}

// lambda = damp_rel * mean(diag H), summed in float64 by one workgroup.
__global__ __launch_bounds__(kThreads) void damp_kernel(const float* __restrict__ H, int n,
                                                        double damp_rel, double* __restrict__ lam) {
  __shared__ double red[kThreads];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kThreads) s += (double)H[(int64_t)i * n + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *lam = damp_rel * (red[0] / (double)n);
}

// perm = identity, or the stable descending order of diag(H): the rank of
// column i is the number of columns with a larger diagonal, or an equal one
// and a smaller index.
__global__ __launch_bounds__(kThreads) void act_order_kernel(const float* __restrict__ H, int n,
                                                             int act_order, int32_t* __restrict__ perm) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (!act_order) {
    if (i < n) perm[i] = i;
    return;
  }
  // NaN keys sort last (as -inf) so that the result is always a permutation.
  __shared__ float d[kThreads];
  float di = i < n ? H[(int64_t)i * n + i] : 0.f;
  if (isnan(di)) di = -INFINITY;
  int rank = 0;
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    __syncthreads();
    const int j = j0 + threadIdx.x;
    const float dj_raw = j < n ? H[(int64_t)j * n + j] : 0.f;
    d[threadIdx.x] = isnan(dj_raw) ? -INFINITY : dj_raw;
    __syncthreads();
    const int lim = min(kThreads, n - j0);
    for (int t = 0; t < lim; ++t) {
      const float dj = d[t];
      rank += (dj > di || (dj == di && j0 + t < i)) ? 1 : 0;
    }
  }
  if (i < n) perm[rank] = i;
}

// A[i][j] = H[q_i][q_j] + lambda * (i == j), q_i = perm[n-1-i]; identity padding.
__global__ __launch_bounds__(kThreads) void build_reversed_kernel(
    const float* __restrict__ H, int n, int np, const int32_t* __restrict__ perm,
    const double* __restrict__ lam, double* __restrict__ A) {
  const int i = blockIdx.x;
  const double l = *lam;
  const int qi = i < n ? min(max(perm[n - 1 - i], 0), n - 1) : 0;
  for (int j = threadIdx.x; j < np; j += kThreads) {
    double v;
    if (i < n && j < n) {
      const int qj = min(max(perm[n - 1 - j], 0), n - 1);
      v = (double)H[(int64_t)qi * n + qj];
      if (i == j) v += l;
    } else {
      v = (i == j) ? 1.0 : 0.0;
    }
    A[(int64_t)i * np + j] = v;
  }
}

// Zero X (the inverse under construction).
__global__ void zero_kernel(double* __restrict__ p, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0;
}

// 1/sqrt(d) in float64: hardware estimate refined by two Newton steps.
__device__ inline double rsqrt_f64(double d) {
  double y = __builtin_amdgcn_rsq(d);
  double h = __builtin_fma(-0.5 * d * y, y, 0.5);
  y = __builtin_fma(y, h, y);
  h = __builtin_fma(-0.5 * d * y, y, 0.5);
  return __builtin_fma(y, h, y);
}

__device__ inline double bcast_lane(double v, int lane) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)u, lane);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)(u >> 32), lane);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Factors and inverts the 64 x 64 diagonal block kb; called by all 256
// threads of a workgroup.
//  Cholesky (wave 0 only; lane r owns row r in registers, columns are
//  broadcast with readlane, so no barrier is needed inside the loop):
//    column j:  y = 1/sqrt(a_jj);  L_rj = a_rj * y (r >= j, so L_jj = sqrt(a_jj));
//               a_rc -= L_rj L_cj  (j < c <= r)
//  Inverse (all 4 waves, wave w owns columns w, w+4, ..., w+60): the columns of
//  V = L^{-1} are independent; V = diag(1/L_jj) T with T = I and, for each row
//  j, rows r > j: T[r][c] -= (L_rj / L_jj) T[j][c].
// S is an LDS copy of the block (pitch kB + 1).  L goes back to A, inv(L_kk)
// to Linv and to X's diagonal block.  A non-positive or non-finite pivot
// leaves L_jj non-finite or zero (NaN then spreads to every later pivot), so
// the first bad pivot is the first row whose L_rr is not a positive finite
// number; it is recorded in *info.
__device__ inline void factor_diag(double* S, double* __restrict__ A, double* __restrict__ X,
                                   double* __restrict__ Linv, int np, int n, int kb,
                                   int32_t* __restrict__ info) {
  constexpr int P = kB + 1;
  const int wave = threadIdx.x >> 6;
  const int r = threadIdx.x & 63;
  const int64_t base = (int64_t)kb * kB * np + (int64_t)kb * kB;
  if (wave == 0) {
    double a[kB];
#pragma unroll
    for (int c = 0; c < kB; ++c) a[c] = c <= r ? S[r * P + c] : 0.0;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const double y = rsqrt_f64(bcast_lane(a[j], j));
      a[j] *= y;
#pragma unroll
      for (int c = j + 1; c < kB; ++c) a[c] = __builtin_fma(-a[j], bcast_lane(a[j], c), a[c]);
    }
#pragma unroll
    for (int c = 0; c < kB; ++c) {
      S[r * P + c] = a[c];
      if (c <= r) A[base + (int64_t)r * np + c] = a[c];
    }
    const double lrr = S[r * P + r];
    const bool bad = !(lrr > 0.0) || !isfinite(lrr) || !(lrr * lrr > 0.0);
    const unsigned long long mask = __ballot(bad && kb * kB + r < n);
    if (r == 0 && mask != 0ull && *info == 0) *info = kb * kB + __builtin_ctzll(mask) + 1;
  }
  __syncthreads();
  const double my_y = 1.0 / S[r * P + r];   // 1 / L_rr
  double v[kB / 4];
#pragma unroll
  for (int i = 0; i < kB / 4; ++i) v[i] = (wave + 4 * i == r) ? 1.0 : 0.0;
#pragma unroll
  for (int j = 0; j < kB; ++j) {
    // keep each step's LDS read inside its step (hoisting all of them spills)
    __asm__ volatile("" ::: "memory");
    const double l = (j < r ? S[r * P + j] : 0.0) * bcast_lane(my_y, j);
#pragma unroll
    for (int i = 0; i < kB / 4; ++i) v[i] = __builtin_fma(-l, bcast_lane(v[i], j), v[i]);
  }
#pragma unroll
  for (int i = 0; i < kB / 4; ++i) {
    const int c = wave + 4 * i;
    const double vv = v[i] * my_y;
    Linv[r * kB + c] = vv;
    X[base + (int64_t)r * np + c] = vv;
  }
}

__global__ __launch_bounds__(kThreads) void potrf_diag_kernel(double* __restrict__ A, double* __restrict__ X,
                                                              double* __restrict__ Linv, int np, int n, int kb,
                                                              int32_t* __restrict__ info) {
  __shared__ double S[kB * (kB + 1)];
  const int64_t base = (int64_t)kb * kB * np + (int64_t)kb * kB;
  for (int e = threadIdx.x; e < kB * kB; e += kThreads) S[(e >> 6) * (kB + 1) + (e & 63)] = A[base + (int64_t)(e >> 6) * np + (e & 63)];
  __syncthreads();
  factor_diag(S, A, X, Linv, np, n, kb, info);
}

__device__ inline void tri_decode(int t, int& ii, int& jj) {
  // lower-triangle order (ii >= jj), row by row
  int r = (int)((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  ii = r;
  jj = t - r * (r + 1) / 2;
}

struct TileLds {
  double As[kB][kB + 1];   // As[row][k]
  double Bs[kB][kB + 1];   // Bs[k][col]
};

// One 64 x 64 output block, K = 64, float64 MFMA 16x16x4, 4 waves of 32 x 32:
//   C = (sub ? C : 0) - / + Aop * (transB ? B^T : B)
// All operands are in LDS before C is written, so C may alias Aop or B.
// If keep != nullptr the result is also left in keep[64][65] (LDS).
__device__ inline void gemm_tile64(TileLds& t, const double* Ap, int64_t lda, const double* Bp, int64_t ldb,
                                   bool transB, double* Cp, int64_t ldc, bool sub, double* keep) {
  const int tid = threadIdx.x;
  for (int e = tid; e < kB * kB; e += kThreads) {
    const int r = e >> 6, c = e & 63;
    t.As[r][c] = Ap[(int64_t)r * lda + c];
    if (transB)
      t.Bs[c][r] = Bp[(int64_t)r * ldb + c];
    else
      t.Bs[r][c] = Bp[(int64_t)r * ldb + c];
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1;
  doublex4 acc[2][2];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) acc[ti][tj] = doublex4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int k4 = 0; k4 < kB / 4; ++k4) {
    const int k = k4 * 4 + (lane >> 4);
    double a[2], b[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) a[ti] = t.As[wr * 32 + ti * 16 + (lane & 15)][k];
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) b[tj] = t.Bs[k][wc * 32 + tj * 16 + (lane & 15)];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
        acc[ti][tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ti], b[tj], acc[ti][tj], 0, 0, 0);
  }
  if (keep) __syncthreads();   // keep aliases As
  // float64 16x16x4 accumulator on gfx950: register r of lane l holds row
  // l/16 + 4*r, column l%16 of the 16x16 block (rows interleaved, unlike the
  // float32 16x16x4 form where lane l holds rows 4*(l/16) .. 4*(l/16)+3).
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wr * 32 + ti * 16 + (lane >> 4) + 4 * r;
        const int col = wc * 32 + tj * 16 + (lane & 15);
        double* p = Cp + (int64_t)row * ldc + col;
        const double v = sub ? (*p - acc[ti][tj][r]) : acc[ti][tj][r];
        *p = v;
        if (keep) keep[row * (kB + 1) + col] = v;
      }
}

// Step kb, first launch: panel L[i, kb] = A[i, kb] inv(L_kk)^T for i > kb
// (blocks 0 .. T-1), and row kb of the inverse X[kb, j] = inv(L_kk) T[kb, j]
// for j < kb (blocks T .. T+kb-1).
__global__ __launch_bounds__(kThreads) void chol_panel_kernel(double* __restrict__ A, double* __restrict__ X,
                                                              const double* __restrict__ Linv, int np, int nbk,
                                                              int kb) {
  __shared__ TileLds t;
  const int T = nbk - kb - 1;
  const int b = blockIdx.x;
  if (b < T) {
    const int bi = kb + 1 + b;
    double* p = A + (int64_t)bi * kB * np + (int64_t)kb * kB;
    gemm_tile64(t, p, np, Linv, kB, true, p, np, false, nullptr);
  } else {
    const int bj = b - T;
    double* p = X + (int64_t)kb * kB * np + (int64_t)bj * kB;
    gemm_tile64(t, Linv, kB, p, np, false, p, np, false, nullptr);
  }
}

// Step kb, second launch: trailing update A[i, j] -= L[i, kb] L[j, kb]^T for
// kb < j <= i (blocks 0 .. S-1, block 0 is the next diagonal block, which the
// same workgroup then factors: wave 0 runs factor_diag_wave on it), and
// T[i, j] -= L[i, kb] X[kb, j] for i > kb, j <= kb (the rest).
__global__ __launch_bounds__(kThreads) void chol_update_kernel(double* __restrict__ A, double* __restrict__ X,
                                                               double* __restrict__ Linv, int np, int n, int nbk,
                                                               int kb, int32_t* __restrict__ info) {
  __shared__ TileLds t;
  const int T = nbk - kb - 1;
  const int S = T * (T + 1) / 2;
  const int b = blockIdx.x;
  if (b < S) {
    int ii, jj;
    tri_decode(b, ii, jj);
    const int bi = kb + 1 + ii, bj = kb + 1 + jj;
    const double* pa = A + (int64_t)bi * kB * np + (int64_t)kb * kB;
    const double* pb = A + (int64_t)bj * kB * np + (int64_t)kb * kB;
    double* pc = A + (int64_t)bi * kB * np + (int64_t)bj * kB;
    double* keep = (b == 0) ? &t.As[0][0] : nullptr;
    gemm_tile64(t, pa, np, pb, np, true, pc, np, true, keep);
    if (b == 0) {
      __syncthreads();
      factor_diag(&t.As[0][0], A, X, Linv, np, n, kb + 1, info);
    }
  } else {
    const int e = b - S;
    const int bi = kb + 1 + e / (kb + 1), bj = e % (kb + 1);
    const double* pa = A + (int64_t)bi * kB * np + (int64_t)kb * kB;
    const double* pb = X + (int64_t)kb * kB * np + (int64_t)bj * kB;
    double* pc = X + (int64_t)bi * kB * np + (int64_t)bj * kB;
    gemm_tile64(t, pa, np, pb, np, false, pc, np, true, nullptr);
  }
}

// U[i][j] = X[n-1-i][n-1-j] for i <= j, 0 below the diagonal (float32).
__global__ __launch_bounds__(kThreads) void write_u_kernel(const double* __restrict__ X, int n, int np,
                                                           float* __restrict__ U) {
  const int i = blockIdx.x;
  for (int j = threadIdx.x; j < n; j += kThreads) {
    U[(int64_t)i * n + j] = i <= j ? (float)X[(int64_t)(n - 1 - i) * np + (n - 1 - j)] : 0.f;
  }
}

struct PrepLayout {
  int64_t np;
  size_t off_A, off_X, off_Linv, off_lam, off_info, total;
};

PrepLayout prep_layout(int64_t n) {
  PrepLayout L;
  L.np = round_up(n, kB);
  const size_t mat = (size_t)L.np * (size_t)L.np * sizeof(double);
  L.off_A = 0;
  L.off_X = align256(L.off_A + mat);
  L.off_Linv = align256(L.off_X + mat);
  L.off_lam = align256(L.off_Linv + (size_t)kB * kB * sizeof(double));
  L.off_info = align256(L.off_lam + sizeof(double));
  L.total = align256(L.off_info + sizeof(int32_t));
  return L;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_prepare_ws_bytes(int64_t n) {
  if (n <= 0) return 0;
  return prep_layout(n).total;
}

extern "C" gptq_status gptq_prepare_hinv(const float* H, int64_t n, float damp_rel, int act_order,
                                         float* U, int32_t* perm, int32_t* info_out, void* ws,
                                         size_t ws_bytes, void* stream) {
  if (info_out) *info_out = 0;
  if (n < 0 || !(damp_rel >= 0.f) || !std::isfinite(damp_rel)) return GPTQ_ERR_INVALID_ARG;
  if (n > (int64_t)1 << 16) return GPTQ_ERR_UNSUPPORTED;
  if (n == 0) return GPTQ_OK;
  if (H == nullptr || U == nullptr || perm == nullptr) return GPTQ_ERR_INVALID_ARG;
  const PrepLayout L = prep_layout(n);
  if (ws == nullptr || ws_bytes < L.total) return GPTQ_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  double* A = reinterpret_cast<double*>(base + L.off_A);
  double* X = reinterpret_cast<double*>(base + L.off_X);
  double* Linv = reinterpret_cast<double*>(base + L.off_Linv);
  double* lam = reinterpret_cast<double*>(base + L.off_lam);
  int32_t* info = reinterpret_cast<int32_t*>(base + L.off_info);
  const int ni = (int)n, np = (int)L.np, nbk = (int)(L.np / kB);

  init_scalars_kernel<<<1, 64, 0, st>>>(info);
  damp_kernel<<<1, kThreads, 0, st>>>(H, ni, (double)damp_rel, lam);
  act_order_kernel<<<(unsigned)ceil_div(n, kThreads), kThreads, 0, st>>>(H, ni, act_order, perm);
  build_reversed_kernel<<<(unsigned)np, kThreads, 0, st>>>(H, ni, np, perm, lam, A);
  zero_kernel<<<2048, kThreads, 0, st>>>(X, (int64_t)np * np);
  GPTQ_TRY_LAUNCH();
  potrf_diag_kernel<<<1, kThreads, 0, st>>>(A, X, Linv, np, ni, 0, info);
  for (int kb = 0; kb < nbk; ++kb) {
    const int T = nbk - kb - 1;
    if (T + kb > 0) chol_panel_kernel<<<(unsigned)(T + kb), kThreads, 0, st>>>(A, X, Linv, np, nbk, kb);
    if (T > 0)
      chol_update_kernel<<<(unsigned)(T * (T + 1) / 2 + T * (kb + 1)), kThreads, 0, st>>>(A, X, Linv, np, ni, nbk,
                                                                                         kb, info);
    GPTQ_TRY_LAUNCH();
  }
  write_u_kernel<<<(unsigned)n, kThreads, 0, st>>>(X, ni, np, U);
  GPTQ_TRY_LAUNCH();
  int32_t h_info = 0;
  GPTQ_TRY_HIP(hipMemcpyAsync(&h_info, info, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  GPTQ_TRY_HIP(hipStreamSynchronize(st));
  if (info_out) *info_out = h_info;
  return h_info == 0 ? GPTQ_OK : GPTQ_ERR_NOT_PD;
}
