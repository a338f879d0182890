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
// with 64 x 64 blocks, interleaved in one loop over block columns kb:
//   potrf_diag(kb)  factor the diagonal block, invert it (one workgroup)
//   trsm(kb)        panel L[i, kb] = A[i, kb] * inv(L_kk)^T        (MFMA f64)
//   syrk(kb)        A[i, j] -= L[i, kb] L[j, kb]^T, kb < j <= i    (MFMA f64)
//   tri_fin(kb)     X[kb, j] = inv(L_kk) T[kb, j], j < kb          (MFMA f64)
//   tri_upd(kb)     T[i, j] -= L[i, kb] X[kb, j], i > kb, j <= kb  (MFMA f64)
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

// Factors the 64 x 64 diagonal block kb in LDS (lower Cholesky), records the
// first bad pivot, writes L_kk back, and writes inv(L_kk) both to the
// workspace slot Linv and to the diagonal block of X.
__global__ __launch_bounds__(kThreads) void potrf_diag_kernel(double* __restrict__ A, double* __restrict__ X,
                                                              double* __restrict__ Linv, int np, int n, int kb,
                                                              int32_t* __restrict__ info) {
  __shared__ double L[kB][kB + 1];
  __shared__ double V[kB][kB + 1];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)kb * kB * np + (int64_t)kb * kB;
  for (int e = tid; e < kB * kB; e += kThreads) {
    const int r = e / kB, c = e % kB;
    L[r][c] = c <= r ? A[base + (int64_t)r * np + c] : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < kB; ++j) {
    if (tid == 0) {
      const double d = L[j][j];
      const int pos = kb * kB + j;
      if (!(d > 0.0) || !isfinite(d)) {
        if (pos < n && *info == 0) *info = pos + 1;
      }
      L[j][j] = sqrt(d);
    }
    __syncthreads();
    const double djj = L[j][j];
    for (int r = j + 1 + tid; r < kB; r += kThreads) L[r][j] /= djj;
    __syncthreads();
    // trailing update of the block: L[r][c] -= L[r][j] L[c][j], j < c <= r
    for (int e = tid; e < kB * kB; e += kThreads) {
      const int r = e / kB, c = e % kB;
      if (c > j && c <= r) L[r][c] -= L[r][j] * L[c][j];
    }
    __syncthreads();
  }
  // inverse by columns: V = L^{-1} (lower), column c solved by forward substitution
  if (tid < kB) {
    const int c = tid;
    for (int r = 0; r < kB; ++r) V[r][c] = 0.0;
    V[c][c] = 1.0 / L[c][c];
    for (int r = c + 1; r < kB; ++r) {
      double s = 0.0;
      for (int p = c; p < r; ++p) s += L[r][p] * V[p][c];
      V[r][c] = -s / L[r][r];
    }
  }
  __syncthreads();
  for (int e = tid; e < kB * kB; e += kThreads) {
    const int r = e / kB, c = e % kB;
    if (c <= r) A[base + (int64_t)r * np + c] = L[r][c];
    Linv[e] = V[r][c];
    X[base + (int64_t)r * np + c] = V[r][c];
  }
}

enum { OP_TRSM = 0, OP_SYRK = 1, OP_TRI_FIN = 2, OP_TRI_UPD = 3 };

__device__ inline void tri_decode(int t, int& ii, int& jj) {
  // lower-triangle order (ii >= jj), row by row
  int r = (int)((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  ii = r;
  jj = t - r * (r + 1) / 2;
}

// One 64 x 64 output block per workgroup, K = 64, float64 MFMA 16x16x4.
//   TRSM:    C = Aop * B^T          (C = A[i,kb], Aop = A[i,kb], B = inv(L_kk))
//   SYRK:    C = C - Aop * B^T      (C = A[i,j], Aop = A[i,kb], B = A[j,kb])
//   TRI_FIN: C = Aop * B            (C = X[kb,j], Aop = inv(L_kk), B = X[kb,j])
//   TRI_UPD: C = C - Aop * B        (C = X[i,j], Aop = A[i,kb], B = X[kb,j])
// All operands are loaded into LDS before C is written, so C may alias B.
template <int OP>
__global__ __launch_bounds__(kThreads) void chol_block_kernel(double* __restrict__ A, double* __restrict__ X,
                                                              const double* __restrict__ Linv, int np, int nbk,
                                                              int kb) {
  int bi, bj;
  if (OP == OP_TRSM) {
    bi = kb + 1 + blockIdx.x;
    bj = kb;
  } else if (OP == OP_SYRK) {
    int ii, jj;
    tri_decode(blockIdx.x, ii, jj);
    bi = kb + 1 + ii;
    bj = kb + 1 + jj;
  } else if (OP == OP_TRI_FIN) {
    bi = kb;
    bj = blockIdx.x;
  } else {
    bi = kb + 1 + blockIdx.x / (kb + 1);
    bj = blockIdx.x % (kb + 1);
  }
  if (bi >= nbk) return;

  const double* Ap;
  int64_t lda;
  const double* Bp;
  int64_t ldb;
  double* Cp;
  bool transB, sub;
  if (OP == OP_TRSM) {
    Ap = A + (int64_t)bi * kB * np + (int64_t)kb * kB; lda = np;
    Bp = Linv; ldb = kB; transB = true; sub = false;
    Cp = A + (int64_t)bi * kB * np + (int64_t)kb * kB;
  } else if (OP == OP_SYRK) {
    Ap = A + (int64_t)bi * kB * np + (int64_t)kb * kB; lda = np;
    Bp = A + (int64_t)bj * kB * np + (int64_t)kb * kB; ldb = np; transB = true; sub = true;
    Cp = A + (int64_t)bi * kB * np + (int64_t)bj * kB;
  } else if (OP == OP_TRI_FIN) {
    Ap = Linv; lda = kB;
    Bp = X + (int64_t)kb * kB * np + (int64_t)bj * kB; ldb = np; transB = false; sub = false;
    Cp = X + (int64_t)kb * kB * np + (int64_t)bj * kB;
  } else {
    Ap = A + (int64_t)bi * kB * np + (int64_t)kb * kB; lda = np;
    Bp = X + (int64_t)kb * kB * np + (int64_t)bj * kB; ldb = np; transB = false; sub = true;
    Cp = X + (int64_t)bi * kB * np + (int64_t)bj * kB;
  }

  __shared__ double As[kB][kB + 1];   // As[row][k]
  __shared__ double Bs[kB][kB + 1];   // Bs[k][col]
  const int tid = threadIdx.x;
  for (int e = tid; e < kB * kB; e += kThreads) {
    const int r = e / kB, c = e % kB;
    As[r][c] = Ap[(int64_t)r * lda + c];
    if (transB)
      Bs[c][r] = Bp[(int64_t)r * ldb + c];
    else
      Bs[r][c] = Bp[(int64_t)r * ldb + c];
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
    for (int ti = 0; ti < 2; ++ti) a[ti] = As[wr * 32 + ti * 16 + (lane & 15)][k];
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) b[tj] = Bs[k][wc * 32 + tj * 16 + (lane & 15)];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
        acc[ti][tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ti], b[tj], acc[ti][tj], 0, 0, 0);
  }
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
        double* p = Cp + (int64_t)row * np + col;
        const double v = acc[ti][tj][r];
        *p = sub ? (*p - v) : v;
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
  for (int kb = 0; kb < nbk; ++kb) {
    potrf_diag_kernel<<<1, kThreads, 0, st>>>(A, X, Linv, np, ni, kb, info);
    const int rest = nbk - kb - 1;
    if (rest > 0) {
      chol_block_kernel<OP_TRSM><<<(unsigned)rest, kThreads, 0, st>>>(A, X, Linv, np, nbk, kb);
      chol_block_kernel<OP_SYRK><<<(unsigned)(rest * (rest + 1) / 2), kThreads, 0, st>>>(A, X, Linv, np, nbk, kb);
    }
    if (kb > 0) chol_block_kernel<OP_TRI_FIN><<<(unsigned)kb, kThreads, 0, st>>>(A, X, Linv, np, nbk, kb);
    if (rest > 0)
      chol_block_kernel<OP_TRI_UPD><<<(unsigned)(rest * (kb + 1)), kThreads, 0, st>>>(A, X, Linv, np, nbk, kb);
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
