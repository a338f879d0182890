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
// with 64 x 64 blocks, in one loop over block columns kb:
//   panel(kb)   L[i, kb] = A[i, kb] inv(L_kk)^T                   (MFMA f64)
//               X[kb, j] = inv(L_kk) T[kb, j], j < kb             (MFMA f64)
//   update      A[i, j] -= sum_p L[i, p] L[j, p]^T                (MFMA f64)
//               T[i, j] -= sum_p L[i, p] X[p, j]                  (MFMA f64)
//               + the workgroup that updates the next diagonal block then
//                 factors and inverts it (16-column leaves, float64 MFMA
//                 between them), overlapping the rest of the trailing update
// where X = L^{-1} is built in place of T (forward substitution by block
// rows).  For large n block columns are taken in groups of four p0 .. p0+3:
// panel(p0 + t), each but the last followed by a narrow update of block
// column and inverse row p0+t+1 alone with panels p0 .. p0+t, then one
// trailing update with all four panels (K = 256) -- the float64 trailing
// matrix is read and written once per group instead of once per block
// column, which cuts the memory traffic that bounds large n.
// Matrices are padded to a multiple of 64 with an identity block.
#include "common.h"

namespace gptq {
namespace {

constexpr int kB = 64;        // Cholesky block
constexpr int kThreads = 256;
constexpr int kUpdateBlocks = 256;  // workgroups of the trailing-update launch (one per CU)
constexpr int kGroupWide = 4;       // block columns per trailing update for large n

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
// Only the lower block triangle (block column <= block row) is written:
// nothing reads A's blocks above the diagonal.
__global__ __launch_bounds__(kThreads) void build_reversed_kernel(
    const float* __restrict__ H, int n, int np, const int32_t* __restrict__ perm,
    const double* __restrict__ lam, double* __restrict__ A) {
  const int i = blockIdx.x;
  const double l = *lam;
  const int qi = i < n ? min(max(perm[n - 1 - i], 0), n - 1) : 0;
  const int jend = (i / kB + 1) * kB;
  for (int j = threadIdx.x; j < jend; j += kThreads) {
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

// 1/sqrt(d) in float64: hardware estimate (relative error below 2^-24,
// measured over random inputs on gfx950) refined by one Newton step (below
// 2^-47).  It sits on the column chain of every diagonal factor; that
// accuracy is far beyond what the float32 U kept at the end can show.
__device__ inline double rsqrt_f64(double d) {
  const double y = __builtin_amdgcn_rsq(d);
  const double h = __builtin_fma(-0.5 * d * y, y, 0.5);
  return __builtin_fma(y, h, y);
}

__device__ inline double bcast_lane(double v, int lane) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)u, lane);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)(u >> 32), lane);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// The 64 x 64 diagonal block: Cholesky factor and its inverse.
//
// The block is split into four 16-column leaves.  Wave 0 factors one leaf at
// a time for all 64 rows (lane = row; the 16 columns live in registers and
// pivot columns are broadcast with readlane, so the rows below the leaf's
// diagonal block come out of the same instructions).  Between leaves all four
// waves apply the leaf's rank-16 update to the remaining blocks with float64
// MFMA.  The inverse X = inv(L) is built by 16 x 16 blocks on the other waves
// while wave 0 factors the next leaf:
//   X_II = inv(L_II)                 (lane = column, forward substitution)
//   X_IJ = -X_II sum_{K=J}^{I-1} L_IK X_KJ   (MFMA, J < I)
// S holds the block (pitch 65) and receives L; Xs (pitch 65) receives X.
// A non-positive or non-finite pivot leaves L_jj non-finite or zero (NaN then
// spreads to every later pivot), so the first bad pivot is the first row whose
// L_rr is not a positive finite number; it is recorded in *info.
// ---------------------------------------------------------------------------
constexpr int kP = kB + 1;    // LDS pitch of the 64 x 64 block buffers

struct FactorLds {
  double yd[kB];              // 1 / L_jj
  double Ts[3][16][17];       // partial sums of the off-diagonal inverse blocks
};

// float64 MFMA 16x16x4 operand/accumulator layouts on gfx950: A element
// (row l%16, k l/16), B element (k l/16, column l%16); accumulator register r
// of lane l holds row l/16 + 4r, column l%16.
__device__ __forceinline__ doublex4 load_c16(const double* C, int ldc, int lane) {
  doublex4 a;
#pragma unroll
  for (int r = 0; r < 4; ++r) a[r] = C[((lane >> 4) + 4 * r) * ldc + (lane & 15)];
  return a;
}

__device__ __forceinline__ void store_c16(double* C, int ldc, doublex4 a, int lane) {
#pragma unroll
  for (int r = 0; r < 4; ++r) C[((lane >> 4) + 4 * r) * ldc + (lane & 15)] = a[r];
}

// acc += (neg ? -A : A) B for 16 x 16 row-major blocks in LDS.
__device__ __forceinline__ doublex4 mm16(doublex4 acc, const double* Ab, int lda, const double* Bb, int ldb,
                                         bool neg, int lane) {
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    const int k = k4 * 4 + (lane >> 4);
    const double a = Ab[(lane & 15) * lda + k];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(neg ? -a : a, Bb[k * ldb + (lane & 15)], acc, 0, 0, 0);
  }
  return acc;
}

// acc += (neg ? -A : A) Bt^T.
__device__ __forceinline__ doublex4 mm16_bt(doublex4 acc, const double* Ab, int lda, const double* Bt, int ldbt,
                                            bool neg, int lane) {
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    const int k = k4 * 4 + (lane >> 4);
    const double a = Ab[(lane & 15) * lda + k];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(neg ? -a : a, Bt[(lane & 15) * ldbt + k], acc, 0, 0, 0);
  }
  return acc;
}

// Wave 0: columns 16Q .. 16Q+15 of S for all rows (right-looking inside the
// leaf); rows above the diagonal are written as zero.
template <int Q>
__device__ __forceinline__ void leaf_factor(double* S, double* yd, int lane) {
  double v[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int c = 16 * Q + jj;
    const double s = S[lane * kP + c];
    v[jj] = c <= lane ? s : 0.0;
  }
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = 16 * Q + jj;
    const double y = rsqrt_f64(bcast_lane(v[jj], j));
    v[jj] *= y;
    yd[j] = y;
#pragma unroll
    for (int cc = jj + 1; cc < 16; ++cc) v[cc] = __builtin_fma(-v[jj], bcast_lane(v[jj], 16 * Q + cc), v[cc]);
  }
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int c = 16 * Q + jj;
    S[lane * kP + c] = c <= lane ? v[jj] : 0.0;
  }
}

// All waves: blocks (I, J) with Q < J <= I get -= L_IQ L_JQ^T.
template <int Q>
__device__ __forceinline__ void leaf_update(double* S, int wave, int lane) {
  int idx = 0;
#pragma unroll
  for (int I = Q + 1; I < 4; ++I)
#pragma unroll
    for (int J = Q + 1; J <= I; ++J, ++idx) {
      if ((idx & 3) != wave) continue;
      double* C = S + 16 * I * kP + 16 * J;
      doublex4 acc = load_c16(C, kP, lane);
      acc = mm16_bt(acc, S + 16 * I * kP + 16 * Q, kP, S + 16 * J * kP + 16 * Q, kP, true, lane);
      store_c16(C, kP, acc, lane);
    }
}

// X_II = inv(L_II): lane & 15 is the column, rows by forward substitution.
template <int I>
__device__ __forceinline__ void leaf_inverse(const double* S, double* Xs, const double* yd, int lane) {
  const int c = lane & 15;
  double x[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    double p0 = rr == c ? 1.0 : 0.0, p1 = 0.0;
#pragma unroll
    for (int k = 0; k < rr; ++k) {
      const double l = S[(16 * I + rr) * kP + 16 * I + k];
      if (k & 1)
        p1 = __builtin_fma(-l, x[k], p1);
      else
        p0 = __builtin_fma(-l, x[k], p0);
    }
    x[rr] = (p0 + p1) * yd[16 * I + rr];
  }
  if (lane < 16) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) Xs[(16 * I + rr) * kP + 16 * I + c] = x[rr];
  }
}

// sum_{K=J}^{I-1} L_IK X_KJ
template <int I, int J>
__device__ __forceinline__ doublex4 inverse_row_sum(const double* S, const double* Xs, int lane) {
  doublex4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int K = J; K < I; ++K) acc = mm16(acc, S + 16 * I * kP + 16 * K, kP, Xs + 16 * K * kP + 16 * J, kP, false, lane);
  return acc;
}

// X_IJ = -X_II T, T (16 x 16, pitch 17) in LDS.
template <int I, int J>
__device__ __forceinline__ void inverse_finish(double* Xs, const double* T, int lane) {
  doublex4 acc = {0.0, 0.0, 0.0, 0.0};
  acc = mm16(acc, Xs + 16 * I * kP + 16 * I, kP, T, 17, true, lane);
  store_c16(Xs + 16 * I * kP + 16 * J, kP, acc, lane);
}

template <int I, int J>
__device__ __forceinline__ void inverse_block(const double* S, double* Xs, double* T, int lane) {
  store_c16(T, 17, inverse_row_sum<I, J>(S, Xs, lane), lane);
  inverse_finish<I, J>(Xs, T, lane);
}

// Factors and inverts the diagonal block kb held in S; all 256 threads.
// inv(L_kk) goes to Linv and to X's diagonal block.
__device__ __forceinline__ void factor_diag(double* S, double* Xs, FactorLds& fx, double* __restrict__ X,
                                            double* __restrict__ Linv, int np, int n, int kb,
                                            int32_t* __restrict__ info) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)kb * kB * np + (int64_t)kb * kB;
  double* T0 = &fx.Ts[0][0][0];
  double* T1 = &fx.Ts[1][0][0];
  double* T2 = &fx.Ts[2][0][0];
  if (wave == 0) leaf_factor<0>(S, fx.yd, lane);
  __syncthreads();
  leaf_update<0>(S, wave, lane);
  __syncthreads();
  if (wave == 0) leaf_factor<1>(S, fx.yd, lane);
  if (wave == 1) leaf_inverse<0>(S, Xs, fx.yd, lane);
  __syncthreads();
  leaf_update<1>(S, wave, lane);
  __syncthreads();
  if (wave == 0) leaf_factor<2>(S, fx.yd, lane);
  if (wave == 1) {
    leaf_inverse<1>(S, Xs, fx.yd, lane);
    inverse_block<1, 0>(S, Xs, T0, lane);
  }
  __syncthreads();
  leaf_update<2>(S, wave, lane);
  __syncthreads();
  if (wave == 0) leaf_factor<3>(S, fx.yd, lane);
  if (wave == 1) leaf_inverse<2>(S, Xs, fx.yd, lane);
  if (wave == 2) store_c16(T0, 17, inverse_row_sum<2, 0>(S, Xs, lane), lane);
  if (wave == 3) store_c16(T1, 17, inverse_row_sum<2, 1>(S, Xs, lane), lane);
  __syncthreads();
  if (wave == 1) inverse_finish<2, 1>(Xs, T1, lane);
  if (wave == 2) inverse_finish<2, 0>(Xs, T0, lane);
  if (wave == 3) leaf_inverse<3>(S, Xs, fx.yd, lane);
  __syncthreads();
  if (wave == 1) inverse_block<3, 0>(S, Xs, T0, lane);
  if (wave == 2) inverse_block<3, 1>(S, Xs, T1, lane);
  if (wave == 3) inverse_block<3, 2>(S, Xs, T2, lane);
  if (wave == 0) {
    const double lrr = S[lane * kP + lane];
    const bool bad = !(lrr > 0.0) || !isfinite(lrr) || !(lrr * lrr > 0.0);
    const unsigned long long mask = __ballot(bad && kb * kB + lane < n);
    if (lane == 0 && mask != 0ull && *info == 0) *info = kb * kB + __builtin_ctzll(mask) + 1;
  }
  __syncthreads();
  // Two elements per thread and store.  The factor itself is not written
  // back: nothing reads the diagonal blocks of L after this point.
  for (int e = threadIdx.x; e < kB * kB / 2; e += kThreads) {
    const int r = e >> 5, c = (e & 31) * 2;
    const double2 xv = {c <= r ? Xs[r * kP + c] : 0.0, c + 1 <= r ? Xs[r * kP + c + 1] : 0.0};
    *reinterpret_cast<double2*>(Linv + r * kB + c) = xv;
    *reinterpret_cast<double2*>(X + base + (int64_t)r * np + c) = xv;
  }
}

struct TileLds {
  double As[kB][kP];   // As[row][k]
  double Bs[kB][kP];   // Bs[k][col]
};

__global__ __launch_bounds__(kThreads) void potrf_diag_kernel(double* __restrict__ A, double* __restrict__ X,
                                                              double* __restrict__ Linv, int np, int n, int kb,
                                                              int32_t* __restrict__ info) {
  __shared__ TileLds t;
  __shared__ FactorLds fx;
  const int64_t base = (int64_t)kb * kB * np + (int64_t)kb * kB;
  for (int e = threadIdx.x; e < kB * kB / 2; e += kThreads) {
    const int r = e >> 5, c = (e & 31) * 2;
    const double2 v = *reinterpret_cast<const double2*>(A + base + (int64_t)r * np + c);
    t.As[r][c] = v.x;
    t.As[r][c + 1] = v.y;
  }
  __syncthreads();
  factor_diag(&t.As[0][0], &t.Bs[0][0], fx, X, Linv, np, n, kb, info);
}

__device__ inline void tri_decode(int t, int& ii, int& jj) {
  // lower-triangle order (ii >= jj), row by row
  int r = (int)((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  ii = r;
  jj = t - r * (r + 1) / 2;
}


// One 64 x 64 output block, K = 64, float64 MFMA 16x16x4, 4 waves of 32 x 32:
//   C = (sub ? C : 0) - / + Aop * (transB ? B^T : B)
// All operands are in LDS before C is written, so C may alias Aop or B.
// If keep != nullptr the result is also left in keep[64][65] (LDS).
__device__ inline void gemm_tile64(TileLds& t, const double* Ap, int64_t lda, const double* Bp, int64_t ldb,
                                   bool transB, double* Cp, int64_t ldc, bool sub, double* keep) {
  const int tid = threadIdx.x;
  // Two elements per load (every operand row starts 16-byte aligned).
  for (int e = tid; e < kB * kB / 2; e += kThreads) {
    const int r = e >> 5, c = (e & 31) * 2;
    const double2 a = *reinterpret_cast<const double2*>(Ap + (int64_t)r * lda + c);
    const double2 b = *reinterpret_cast<const double2*>(Bp + (int64_t)r * ldb + c);
    t.As[r][c] = a.x;
    t.As[r][c + 1] = a.y;
    if (transB) {
      t.Bs[c][r] = b.x;
      t.Bs[c + 1][r] = b.y;
    } else {
      t.Bs[r][c] = b.x;
      t.Bs[r][c + 1] = b.y;
    }
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
// (tiles 0 .. T-1; also written transposed to Lt[lt_row0 + k][i], the
// row-major B operand of the trailing update) and row kb of the inverse X[kb, j] = inv(L_kk) T[kb, j]
// for j < kb (tiles T .. T+kb-1), four workgroups per 64 x 64 tile.  A
// workgroup owns 16 output rows of a panel tile (which read only those rows)
// or 16 output columns of an inverse-row tile (which read only those
// columns), so results go back in place without races; each wave computes
// one 16 x 16 block with 16 float64 MFMAs.
__global__ __launch_bounds__(kThreads) void chol_panel_kernel(double* __restrict__ A, double* __restrict__ X,
                                                              const double* __restrict__ Linv,
                                                              double* __restrict__ Lt, int np, int nbk, int kb,
                                                              int lt_row0) {
  __shared__ double Ls[kB][kP];      // inv(L_kk)
  __shared__ double Ps[kB][17];      // the tile's 16 rows (transposed) or 16 columns, [k][16]
  const int T = nbk - kb - 1;
  const int tile = (int)(blockIdx.x >> 2), part = (int)(blockIdx.x & 3);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool panel = tile < T;
  double* p = panel ? A + (int64_t)(kb + 1 + tile) * kB * np + (int64_t)kb * kB + (int64_t)part * 16 * np
                    : X + (int64_t)kb * kB * np + (int64_t)(tile - T) * kB + part * 16;
  for (int e = tid; e < kB * kB / 2; e += kThreads) {
    const double2 v = reinterpret_cast<const double2*>(Linv)[e];
    Ls[e >> 5][(e & 31) * 2] = v.x;
    Ls[e >> 5][(e & 31) * 2 + 1] = v.y;
  }
  for (int e = tid; e < kB * 16; e += kThreads) {
    if (panel) {
      const int r = e >> 6, k = e & 63;
      Ps[k][r] = p[(int64_t)r * np + k];
    } else {
      const int k = e >> 4, c = e & 15;
      Ps[k][c] = p[(int64_t)k * np + c];
    }
  }
  __syncthreads();
  // Two accumulators (even and odd k4) halve the dependent MFMA chain.
  doublex4 acc2[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
#pragma unroll
  for (int k4 = 0; k4 < kB / 4; ++k4) {
    const int k = k4 * 4 + (lane >> 4);
    // panel: C = P Linv^T (A element P[row][k], B element Linv[col][k]);
    // inverse row: C = Linv P (A element Linv[row][k], B element P[k][col]).
    const double a = panel ? Ps[k][lane & 15] : Ls[wave * 16 + (lane & 15)][k];
    const double b = panel ? Ls[wave * 16 + (lane & 15)][k] : Ps[k][lane & 15];
    acc2[k4 & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc2[k4 & 1], 0, 0, 0);
  }
  const doublex4 acc = acc2[0] + acc2[1];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (lane >> 4) + 4 * r, col = lane & 15;
    if (panel) {
      p[(int64_t)row * np + wave * 16 + col] = acc[r];
      Lt[(int64_t)(lt_row0 + wave * 16 + col) * np + (kb + 1 + tile) * kB + part * 16 + row] = acc[r];
    } else
      p[(int64_t)(wave * 16 + row) * np + col] = acc[r];
  }
}

// The trailing update with panels p0 .. kl = p0 + P - 1 (P = 1 or 2), next =
// kl + 1.  Full mode: "SYRK" tiles A[i, j] -= sum_p L[i, p] L[j, p]^T for
// next <= j <= i and "inverse" tiles T[i, j] -= sum_p L[i, p] X[p, j] for
// i >= next, j <= kl (only panels p >= j: X is lower triangular).  Narrow
// mode (P = 1): only block column next (SYRK tiles (i, next), i >= next) and
// inverse row next (tiles (next, j), j <= kl) -- what panel(next) reads.
// Tile 0 is the diagonal block (next, next); workgroup 0 updates it and then
// factors and inverts it with factor_diag.  Every wave of the other
// workgroups owns a contiguous range of half tiles (32 rows x 64 columns) and
// runs each on its own: operands go from global memory (mostly L2) straight
// into MFMA registers in 16-column-deep chunks, the next chunk in flight
// while the current one multiplies, so no wave waits for another and loads,
// stores and MFMAs of one wave overlap.  No tile reads what another tile of
// the launch writes.  An inverse tile T[i, j] with j >= p0 is touched for the
// first time by this launch (it starts from zero).
struct UpdPlan {
  int p0, P, next, T, S, total;
  bool narrow;
};

__host__ __device__ inline UpdPlan upd_plan(int nbk, int p0, int P, bool narrow) {
  UpdPlan u;
  u.p0 = p0;
  u.P = P;
  u.next = p0 + P;
  u.narrow = narrow;
  u.T = nbk - u.next;
  u.S = narrow ? u.T : u.T * (u.T + 1) / 2;
  u.total = u.S + (narrow ? u.next : u.T * u.next);
  return u;
}

// Tile t of the plan: block row / column, SYRK or inverse.
__device__ inline void upd_tile(const UpdPlan& u, int t, int& bi, int& bj, bool& syrk) {
  syrk = t < u.S;
  if (syrk) {
    if (u.narrow) {
      bi = u.next + t;
      bj = u.next;
    } else {
      int ii, jj;
      tri_decode(t, ii, jj);
      bi = u.next + ii;
      bj = u.next + jj;
    }
  } else {
    const int e = t - u.S;
    if (u.narrow) {
      bi = u.next;
      bj = e;
    } else {
      bi = u.next + e / u.next;
      bj = e % u.next;
    }
  }
}

// Full-mode tiles in band order: bands of kBand block columns, and within a
// band the columns in order, each column's tiles top to bottom -- first the
// SYRK triangle (band b: columns next + b kBand .., each from its diagonal
// tile down), then the inverse rectangle (band b: columns b kBand .., rows
// next .. nbk-1).  Work is handed out in contiguous ranges of this order,
// one range of it per XCD: the waves of an XCD then work on the columns of
// one band at once, each a short run down one column, so a column's B block
// is read by the waves on that column and a row's A half by the waves on the
// band's columns at about the same time, and both stay in that XCD's L2
// between those uses.  Tile 0 is still the diagonal block.  The walk starts
// with a loop over the bands and then steps one tile at a time.
constexpr int kBand = 8;
struct BandWalk {
  int t;          // tile index of the current position
  int b, c, r;    // band, column within the band, row within the band's rows
  bool syrk;
};

__device__ inline int band_width(int b, int cols) { return min(kBand, cols - b * kBand); }

// SYRK band b of a T x T lower triangle: R = T - b kBand rows, column c
// (c < wb) holds rows c .. R-1.
__device__ inline int syrk_band_tiles(int T, int b) {
  const int R = T - b * kBand, wb = min(kBand, R);
  return wb * R - wb * (wb - 1) / 2;
}

__device__ inline void band_start(const UpdPlan& u, int t, BandWalk& w) {
  w.t = t;
  if (t < u.S) {
    w.syrk = true;
    int b = 0, e = t;
    while (e >= syrk_band_tiles(u.T, b)) e -= syrk_band_tiles(u.T, b++);
    const int R = u.T - b * kBand;
    int c = 0;
    while (e >= R - c) e -= R - c++;
    w.b = b;
    w.c = c;
    w.r = c + e;
  } else {
    w.syrk = false;
    int e = t - u.S, b = 0;
    while (e >= u.T * band_width(b, u.next)) e -= u.T * band_width(b++, u.next);
    w.b = b;
    w.c = e / u.T;
    w.r = e % u.T;
  }
}

__device__ inline void band_step(const UpdPlan& u, BandWalk& w) {
  ++w.t;
  if (w.syrk) {
    const int R = u.T - w.b * kBand;
    if (++w.r < R) return;
    if (++w.c < band_width(w.b, u.T)) {
      w.r = w.c;
      return;
    }
    w.c = w.r = 0;
    if (++w.b * kBand < u.T) return;
    w.syrk = false;   // on to the inverse rectangle
    w.b = 0;
    return;
  }
  if (++w.r < u.T) return;
  w.r = 0;
  if (++w.c < band_width(w.b, u.next)) return;
  w.c = 0;
  ++w.b;
}

__device__ inline void band_tile(const UpdPlan& u, const BandWalk& w, int& bi, int& bj, bool& syrk) {
  syrk = w.syrk;
  if (w.syrk) {
    bi = u.next + w.b * kBand + w.r;
    bj = u.next + w.b * kBand + w.c;
  } else {
    bi = u.next + w.r;
    bj = w.b * kBand + w.c;
  }
}

// Half tiles per workgroup of the trailing update (one per wave at a time).
constexpr int kUpdWaves = kThreads / 64;

// Workgroups for an update launch: workgroup 0 plus enough for about one half
// tile per wave, at most one workgroup per CU.
inline int update_grid(const UpdPlan& u) {
  const int units = 2 * (u.total - 1);
  return 1 + std::min((units + kUpdWaves - 1) / kUpdWaves, kUpdateBlocks - 1);
}

__global__ __launch_bounds__(kThreads) void chol_update_kernel(double* __restrict__ A, double* __restrict__ X,
                                                               double* __restrict__ Linv,
                                                               const double* __restrict__ Lt, int np, int n, int nbk,
                                                               int p0, int P, int narrow, int32_t* __restrict__ info) {
  __shared__ TileLds tl;
  __shared__ FactorLds fx;
  const UpdPlan up = upd_plan(nbk, p0, P, narrow != 0);
  if (blockIdx.x == 0) {
    // Diagonal block (next, next) -= sum_p L[next, p] L[next, p]^T, then factor.
    double* pc = A + (int64_t)up.next * kB * np + (int64_t)up.next * kB;
    for (int p = 0; p < P; ++p) {
      const double* pa = A + (int64_t)up.next * kB * np + (int64_t)(p0 + p) * kB;
      if (p > 0) __syncthreads();   // the previous product's LDS reads are done
      gemm_tile64(tl, pa, np, pa, np, true, pc, np, true, p + 1 == P ? &tl.As[0][0] : nullptr);
    }
    __syncthreads();
    factor_diag(&tl.As[0][0], &tl.Bs[0][0], fx, X, Linv, np, n, up.next, info);
    return;
  }
  // Half tile u covers tile u/2 (tiles 1 .. total-1), rows 32*(u%2) .. +31.
  // Workgroups are dispatched to the 8 XCDs round-robin (workgroup b on XCD
  // b mod 8); the workers of one XCD take consecutive ranges, so each XCD
  // works on one band of block rows and its L2 holds that band's panel rows
  // instead of the whole panel.
  const int lane = threadIdx.x & 63;
  const int G = (int)gridDim.x, xcd = (int)blockIdx.x & 7, slot = (int)blockIdx.x >> 3;
  int before = 0;
  for (int y = 0; y < xcd; ++y) before += (G - y + 7) / 8 - (y == 0 ? 1 : 0);
  const int worker = before + slot - (xcd == 0 ? 1 : 0);
  const int gw = worker * kUpdWaves + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nw = ((int)gridDim.x - 1) * kUpdWaves;
  const int units = 2 * (up.total - 1);
  const int per = (units + nw - 1) / nw;
  const int u_lo = 2 + gw * per;
  const int u_hi = min(2 + units, u_lo + per);
  if (u_lo >= u_hi) return;
  // float64 MFMA 16x16x4: A element (row l%16, k l/16), B element (k l/16,
  // column l%16), accumulator register r of lane l: row l/16 + 4r, column
  // l%16.  The contraction index and the output columns are permuted so that
  // every load and store is 16 bytes wide: MFMA step s (0..15) of a 64-deep
  // panel with lane quarter q = l/16 stands for k = 8*(s/2) + 2q + s%2 (a
  // lane's two steps 2j, 2j+1 read one adjacent pair of k of its A row), and
  // column block cb (0..3) with MFMA column c stands for tile column
  // 32*(cb/2) + 2c + cb%2 (blocks 2p and 2p+1 read one adjacent pair of
  // columns of a B row and of a C row).  B is row-major over k for both kinds
  // of tile: Lt[k][j] for a SYRK tile, X[p0 rows + k][j] for an inverse tile.
  const int q = lane >> 4, c16 = lane & 15;
  constexpr int kChunk = 4;                    // MFMA steps per chunk (16 of k)
  // One chunk: a[rb][jj] = A row rb*16 + c16 at the k pair of steps 2jj,
  // 2jj+1; b[ss][pp] = B row of step ss at columns 32pp + 2*c16 + 0..1.
  struct Chunk {
    double2 a[2][kChunk / 2];
    double2 b[kChunk][2];
  };
  auto load_chunk = [&](Chunk& ck, const double* ua, const double* ub, int ch) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int jj = 0; jj < kChunk / 2; ++jj) {
        const int k = 8 * (ch * kChunk / 2 + jj) + 2 * q;
        ck.a[rb][jj] = *reinterpret_cast<const double2*>(ua + (int64_t)(rb * 16 + c16) * np + k);
      }
#pragma unroll
    for (int ss = 0; ss < kChunk; ++ss)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int st = ch * kChunk + ss;
        const int k = 8 * (st >> 1) + 2 * q + (st & 1);
        ck.b[ss][pp] = *reinterpret_cast<const double2*>(ub + (int64_t)k * np + 32 * pp + 2 * c16);
      }
  };
  // Unit u's operands from its first usable panel on: A rows of the half
  // tile, the B block (row-major over k, leading dimension np), the C rows,
  // the number of 16-deep chunks, and whether C starts from zero.
  // Full mode walks the band order from the first tile of the range.
  BandWalk walk;
  if (!up.narrow) band_start(up, u_lo >> 1, walk);
  auto unit_ref = [&](int u, const double*& ua, const double*& ub, double*& uc, int& nch, bool& first) {
    int bi, bj;
    bool syrk;
    if (up.narrow) {
      upd_tile(up, u >> 1, bi, bj, syrk);
    } else {
      while (walk.t < (u >> 1)) band_step(up, walk);
      band_tile(up, walk, bi, bj, syrk);
    }
    const int pstart = syrk ? 0 : max(0, bj - p0);   // X[p, bj] = 0 for panels p < bj
    if (syrk) {
      ub = Lt + (int64_t)pstart * kB * np + (int64_t)bj * kB;
      uc = A + (int64_t)bi * kB * np + (int64_t)bj * kB;
    } else {
      ub = X + (int64_t)(p0 + pstart) * kB * np + (int64_t)bj * kB;
      uc = X + (int64_t)bi * kB * np + (int64_t)bj * kB;
    }
    ua = A + ((int64_t)bi * kB + (u & 1) * 32) * np + (int64_t)(p0 + pstart) * kB;
    uc += (int64_t)(u & 1) * 32 * np;
    nch = (P - pstart) * (kB / (4 * kChunk));
    first = !syrk && bj >= p0;
  };
  Chunk ck[2];
  const double *pa, *pb;
  double* pc;
  int nch;
  bool first;
  unit_ref(u_lo, pa, pb, pc, nch, first);
  load_chunk(ck[0], pa, pb, 0);
  for (int u = u_lo; u < u_hi; ++u) {
    doublex4 acc[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = doublex4{0.0, 0.0, 0.0, 0.0};
    // The next unit's first chunk is loaded during this unit's last one (the
    // last unit loads its own first chunk again, which is never used).
    const double *na, *nb;
    double* nc;
    int nnch;
    bool nfirst;
    unit_ref(u + 1 < u_hi ? u + 1 : u, na, nb, nc, nnch, nfirst);
    auto step = [&](Chunk& cur, Chunk& nxt, int ch) {
      if (ch + 1 < nch)
        load_chunk(nxt, pa, pb, ch + 1);
      else
        load_chunk(nxt, na, nb, 0);
#pragma unroll
      for (int ss = 0; ss < kChunk; ++ss)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const double av = (ss & 1) ? cur.a[rb][ss >> 1].y : cur.a[rb][ss >> 1].x;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const double bv = (cb & 1) ? cur.b[ss][cb >> 1].y : cur.b[ss][cb >> 1].x;
            acc[rb][cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[rb][cb], 0, 0, 0);
          }
        }
    };
    // nch is even (4 per panel): chunks alternate between the two named
    // buffers, so no register array is indexed at run time.
    for (int ch = 0; ch < nch; ch += 2) {
      step(ck[0], ck[1], ch);
      step(ck[1], ck[0], ch + 1);
    }
    // C in the accumulator layout, read after the products (so that the
    // operands, the accumulators and C never hold registers at once):
    // cv[rb][pp][r] = row rb*16 + q + 4r, columns 32pp + 2*c16 + 0..1 (column
    // blocks 2pp, 2pp+1).  An inverse tile first touched here has its old
    // contents (X is never cleared as a whole) read but replaced by zero.
    double2 cv[2][2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          cv[rb][pp][r] =
              *reinterpret_cast<const double2*>(pc + (int64_t)(rb * 16 + q + 4 * r) * np + 32 * pp + 2 * c16);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double2 c = cv[rb][pp][r];
          const double c0 = first ? 0.0 : c.x, c1 = first ? 0.0 : c.y;
          *reinterpret_cast<double2*>(pc + (int64_t)(rb * 16 + q + 4 * r) * np + 32 * pp + 2 * c16) =
              double2{c0 - acc[rb][2 * pp][r], c1 - acc[rb][2 * pp + 1][r]};
        }
    pa = na;
    pb = nb;
    pc = nc;
    nch = nnch;
    first = nfirst;
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
  size_t off_A, off_X, off_Linv, off_Lt, off_lam, off_info, total;
};

PrepLayout prep_layout(int64_t n) {
  PrepLayout L;
  L.np = round_up(n, kB);
  const size_t mat = (size_t)L.np * (size_t)L.np * sizeof(double);
  L.off_A = 0;
  L.off_X = align256(L.off_A + mat);
  L.off_Linv = align256(L.off_X + mat);
  L.off_Lt = align256(L.off_Linv + (size_t)kB * kB * sizeof(double));
  L.off_lam = align256(L.off_Lt + (size_t)kGroupWide * kB * (size_t)L.np * sizeof(double));
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
  double* Lt = reinterpret_cast<double*>(base + L.off_Lt);
  double* lam = reinterpret_cast<double*>(base + L.off_lam);
  int32_t* info = reinterpret_cast<int32_t*>(base + L.off_info);
  const int ni = (int)n, np = (int)L.np, nbk = (int)(L.np / kB);

  init_scalars_kernel<<<1, 64, 0, st>>>(info);
  damp_kernel<<<1, kThreads, 0, st>>>(H, ni, (double)damp_rel, lam);
  act_order_kernel<<<(unsigned)ceil_div(n, kThreads), kThreads, 0, st>>>(H, ni, act_order, perm);
  build_reversed_kernel<<<(unsigned)np, kThreads, 0, st>>>(H, ni, np, perm, lam, A);
  GPTQ_TRY_LAUNCH();
  potrf_diag_kernel<<<1, kThreads, 0, st>>>(A, X, Linv, np, ni, 0, info);
  auto panel = [&](int kb, int lt_row0) {
    const int T = nbk - kb - 1;
    if (T + kb > 0)
      chol_panel_kernel<<<(unsigned)(4 * (T + kb)), kThreads, 0, st>>>(A, X, Linv, Lt, np, nbk, kb, lt_row0);
  };
  auto update = [&](int p0, int P, bool narrow) {
    const UpdPlan u = upd_plan(nbk, p0, P, narrow);
    chol_update_kernel<<<(unsigned)update_grid(u), kThreads, 0, st>>>(A, X, Linv, Lt, np, ni, nbk, p0, P,
                                                                      narrow ? 1 : 0, info);
  };
  // Groups of block columns pay once the float64 trailing matrix outgrows the
  // 256 MB last-level cache (padded n >= 6144); below that the update is
  // latency-bound and each narrow launch only adds a step (4096 wide, pairs:
  // 2.57 -> 2.77 ms), so every block column is its own step.  A group of g
  // columns p0 .. p0+g-1: panel(p0 + t) for t = 0 .. g-1, each but the last
  // followed by the narrow update of block column and inverse row p0+t+1
  // with the panels p0 .. p0+t, then one trailing update with all g panels.
  const int group = np >= 6144 ? kGroupWide : 1;
  for (int p0 = 0; p0 < nbk;) {
    const int gsz = std::min(group, nbk - p0);
    for (int t = 0; t < gsz; ++t) {
      panel(p0 + t, t * kB);
      if (t + 1 < gsz) update(p0, t + 1, true);
    }
    if (p0 + gsz < nbk) update(p0, gsz, false);
    p0 += gsz;
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
