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
// float32.  Matrices of r columns (L, K, Omega and the internal Y) are
// row-major n x r.  The n^2 r products (H L and the downdate H - Z Z^T) run
// on the float64 matrix cores; the r x r Cholesky factor and the row-wise
// triangular solves are register-resident single-wave kernels; the m n r
// compensation product is a float64 VALU tile kernel.  Products split over K
// are summed in a fixed order (results do not depend on timing).
#include "common.h"

namespace gptq {
namespace {

constexpr int kR = GPTQ_LOWRANK_MAX_RANK;  // column tile = the largest rank
constexpr int kThreads = 256;
constexpr int kTP = 64;                    // output rows per workgroup
constexpr int kTK = 32;                    // K per LDS stage
constexpr int kPitch = kTP + 4;            // doubles per LDS row (32-byte aligned rows)
constexpr int kTargetBlocks = 512;         // workgroups the matrix-core products aim for
constexpr int kCompensationBlocks = 1024;  // and the compensation product
constexpr int kRefineBlocks = 768;         // and the refinement's gradient product

static_assert(kR == 64, "the tile shapes assume a 64-column rank tile");

// The compensation product Out(p, a) = sum_k D(p, k) B(k, a): D = W - W^
// (formed on the fly from the codes in original column order and the group
// of each column), B = K.
struct TallArgs {
  const void* A;          // W (m x n, leading dimension lda)
  int64_t lda;
  const uint8_t* codes;   // m x n, original column order
  const float* scales;    // m x G
  const uint8_t* zeros;   // m x G
  int64_t G, group;
  const int32_t* gidx;    // group of column k (< G), or NULL: k / group (0 when group is 0)
  const double* B;        // K x r float64, row-major (leading dimension ldb)
  int64_t ldb;
  int64_t P, K, r;
  int64_t kchunk;      // K per split (multiple of kTK)
  double* part;        // splits x P x kR
};

template <int DT>
__device__ inline double w_elem(const void* W, int64_t i) {
  return static_cast<double>(load_as_f32<DT>(W, i));
}

// As[kk][pp] = D(p0 + pp, k0 + kk) = W[p][k] - s_g(k) (c - z_g(k)): exactly the
// float64 difference of the stored weight and its dequantized value (s is
// float32 and c - z a small integer, so s (c - z) is exact); 0 outside.
template <int DT>
__device__ inline void load_a_stage(const TallArgs& a, double (*As)[kPitch], int64_t p0, int64_t k0, int tid) {
  const int kk = tid & 31;
#pragma unroll
  for (int it = 0; it < kTP / 8; ++it) {
    const int pp = (tid >> 5) + 8 * it;
    const int64_t p = p0 + pp, k = k0 + kk;
    double v = 0.0;
    if (p < a.P && k < a.K) {
      const int64_t g = a.gidx ? static_cast<int64_t>(a.gidx[k]) : (a.group ? k / a.group : 0);
      const double s = static_cast<double>(a.scales[p * a.G + g]);
      const double c = static_cast<double>(a.codes[p * a.K + k]);
      const double z = static_cast<double>(a.zeros[p * a.G + g]);
      v = w_elem<DT>(a.A, p * a.lda + k) - s * (c - z);
    }
    As[kk][pp] = v;
  }
}

// part[s][p][a] = sum over split s's K range of D(p, k) B(k, a), for one
// 64-row tile (blockIdx.x) and one split (blockIdx.y): 4 x 4 outputs per
// thread, K staged 32 deep through LDS.
template <int DT>
__global__ __launch_bounds__(kThreads) void compensation_kernel(TallArgs a) {
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
    load_a_stage<DT>(a, As, p0, k0, tid);
    {
      const int col = tid & 63;
#pragma unroll
      for (int it = 0; it < kTK / 4; ++it) {
        const int kk = (tid >> 6) + 4 * it;
        const int64_t k = k0 + kk;
        double v = 0.0;
        if (k < kend && col < a.r) v = a.B[k * a.ldb + col];
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

// The same product on the matrix cores for A(p, k) = S[k][p] (S and B float32
// or float64, widened exactly): float64 MFMA 16x16x4 (A element (row l%16,
// k l/16), B element (k l/16, column l%16), accumulator register i of lane l
// at row l/16 + 4i, column l%16).  A workgroup owns kMP rows and all kR
// columns; its four waves take every fourth 4-deep K step of the split, keep
// kDepth steps of operands in flight, and are summed through LDS in wave
// order at the end.
constexpr int kMP = 32;                   // rows per workgroup
constexpr int kDepth = 4;                 // K steps in flight per wave
constexpr int kMChunk = 16 * kDepth;      // K granularity of a split

template <typename ST, typename BT = double>
__global__ __launch_bounds__(kThreads) void tall_mfma_kernel(const ST* __restrict__ S, int64_t lds_,
                                                             const BT* __restrict__ B, int64_t ldb, int64_t P,
                                                             int64_t K, int r, int64_t kchunk,
                                                             double* __restrict__ part) {
  __shared__ double red[3][kMP][kR + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kl = lane >> 4, cl = lane & 15;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kMP;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * kchunk;
  const int64_t kend = kbeg + kchunk < K ? kbeg + kchunk : K;
  const int64_t kw = kbeg + 4 * wave + kl;       // this lane's K index in step 0
  const int nst = kbeg + 4 * wave < kend ? static_cast<int>((kend - kbeg - 4 * wave + 15) / 16) : 0;
  const int64_t pa = p0 + cl, pb = p0 + 16 + cl;
  const bool pa_in = pa < P, pb_in = pb < P;
  bool c_in[4];
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) c_in[tj] = 16 * tj + cl < r;
  double a0[kDepth], a1[kDepth], b[kDepth][4];
  doublex4 acc[2][4];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) acc[ti][tj] = doublex4{0.0, 0.0, 0.0, 0.0};

#define GPTQ_TALL_LOAD(d, step)                                                     \
  do {                                                                              \
    const int64_t k_ = kw + 16 * static_cast<int64_t>(step);                       \
    const bool kin_ = k_ < kend;                                                    \
    a0[d] = (kin_ && pa_in) ? static_cast<double>(S[k_ * lds_ + pa]) : 0.0;        \
    a1[d] = (kin_ && pb_in) ? static_cast<double>(S[k_ * lds_ + pb]) : 0.0;        \
    _Pragma("unroll") for (int tj = 0; tj < 4; ++tj)                                \
      b[d][tj] = (kin_ && c_in[tj]) ? static_cast<double>(B[k_ * ldb + 16 * tj + cl]) : 0.0; \
  } while (0)

#pragma unroll
  for (int d = 0; d < kDepth; ++d) GPTQ_TALL_LOAD(d, d);
  for (int s0 = 0; s0 < nst; s0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        acc[0][tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0[d], b[d][tj], acc[0][tj], 0, 0, 0);
        acc[1][tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1[d], b[d][tj], acc[1][tj], 0, 0, 0);
      }
      GPTQ_TALL_LOAD(d, s0 + d + kDepth);
    }
  }
#undef GPTQ_TALL_LOAD

  if (wave > 0) {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 4; ++tj)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][16 * ti + kl + 4 * i][16 * tj + cl] = acc[ti][tj][i];
  }
  __syncthreads();
  if (wave == 0) {
    double* out = part + static_cast<int64_t>(blockIdx.y) * P * kR;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * ti + kl + 4 * i;
        const int64_t p = p0 + row;
        if (p >= P) continue;
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
          const int col = 16 * tj + cl;
          double v = acc[ti][tj][i];
          v += red[0][row][col];
          v += red[1][row][col];
          v += red[2][row][col];
          out[p * kR + col] = v;
        }
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

// One workgroup of four waves: G (r x r, leading dimension r, lower triangle
// used) = C C^T (Cholesky, lower), blocked by 16-column panels with the
// matrix in LDS (rows and columns past r are those of the identity).  Panel
// p: wave 0 factors columns 16p .. 16p+15 of every row (lane i = row i,
// the panel in registers; the pivot and the entries of the finished column
// come from their lanes by readlane); then the four waves subtract the panel
// product from the trailing lower 16 x 16 blocks on the float64 matrix cores
// (MFMA 16x16x4: A element (row l%16, k l/16), B element (k l/16, column
// l%16), accumulator register q of lane l at row l/16 + 4q, column l%16).
// Writes C (kR x kR, zero above the diagonal and past r) and Dinv, the
// inverses of C's four 16 x 16 diagonal blocks (identity past r; thread
// 16 b + c builds column c of block b by forward substitution).  A pivot that
// is not a positive finite number sets *flag to 1 (reset clears it first).
constexpr int kMaxGramSplits = 32;  // K splits of the r x r Gram products
constexpr int kBlk = 16;            // panel and diagonal block size
constexpr int kNBlk = kR / kBlk;

__device__ __forceinline__ double lane_value(double v, int lane) {
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(__double2loint(v)), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(__double2hiint(v)), lane);
  return __hiloint2double(hi, lo);
}

// Panel P of the factorization, run by one wave (lane i = row i).
template <int P>
__device__ __forceinline__ void factor_panel(double (*Gs)[kR + 1], int i, int& bad) {
  constexpr int c0 = P * kBlk;
  double g[kBlk];
#pragma unroll
  for (int k = 0; k < kBlk; ++k) g[k] = Gs[i][c0 + k];
#pragma unroll
  for (int k = 0; k < kBlk; ++k) {
    const double d = lane_value(g[k], c0 + k);
    double c = 1.0;
    if (d > 0.0 && d < INFINITY) c = sqrt(d);
    else bad = 1;
    const double lik = i == c0 + k ? c : (i > c0 + k ? g[k] / c : 0.0);
    g[k] = lik;
#pragma unroll
    for (int j = k + 1; j < kBlk; ++j) g[j] = __builtin_fma(-lik, lane_value(lik, c0 + j), g[j]);
  }
#pragma unroll
  for (int k = 0; k < kBlk; ++k)
    if (c0 + k <= i) Gs[i][c0 + k] = g[k];
}

// Trailing update after panel P: every lower 16 x 16 block (bi, bj) with
// bi >= bj > P loses panel(bi) panel(bj)^T; block t of the list goes to wave
// t mod 4.
template <int P>
__device__ __forceinline__ void trailing_update(double (*Gs)[kR + 1], int wave, int lane) {
  constexpr int c0 = P * kBlk;
  constexpr int T = kNBlk - 1 - P;
  const int lr = lane & 15, lq = lane >> 4;
  int t = 0;
#pragma unroll
  for (int bi = P + 1; bi < kNBlk; ++bi)
#pragma unroll
    for (int bj = P + 1; bj <= bi; ++bj, ++t) {
      if (t % 4 != wave) continue;
      doublex4 acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = Gs[kBlk * bi + lq + 4 * q][kBlk * bj + lr];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const double av = -Gs[kBlk * bi + lr][c0 + 4 * s4 + lq];
        const double bv = Gs[kBlk * bj + lr][c0 + 4 * s4 + lq];
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) Gs[kBlk * bi + lq + 4 * q][kBlk * bj + lr] = acc[q];
    }
  (void)T;
}

template <int P>
__device__ __forceinline__ void cholesky_panels(double (*Gs)[kR + 1], int tid, int& bad) {
  const int wave = tid >> 6, lane = tid & 63;
  if (wave == 0) factor_panel<P>(Gs, lane, bad);
  __syncthreads();
  if constexpr (P + 1 < kNBlk) {
    trailing_update<P>(Gs, wave, lane);
    __syncthreads();
    cholesky_panels<P + 1>(Gs, tid, bad);
  }
}

__global__ __launch_bounds__(kThreads) void small_cholesky_kernel(const double* __restrict__ G, int r,
                                                                  double* __restrict__ C, double* __restrict__ Dinv,
                                                                  int32_t* __restrict__ flag, int reset) {
  __shared__ double Gs[kR][kR + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e < kR * kR; e += kThreads) {
    const int a = e / kR, b = e % kR;
    Gs[a][b] = a < r ? (b <= a ? G[a * r + b] : 0.0) : (a == b ? 1.0 : 0.0);
  }
  __syncthreads();
  int bad = 0;  // meaningful in wave 0 (every lane of it sees the same pivots)
  cholesky_panels<0>(Gs, tid, bad);
  for (int e = tid; e < kR * kR; e += kThreads) {
    const int i = e / kR, j = e % kR;
    C[e] = (i < r && j <= i) ? Gs[i][j] : 0.0;
  }
  if (tid < kR) {
    const int b0 = (tid / kBlk) * kBlk, c = tid % kBlk;
    double x[kBlk];
#pragma unroll
    for (int t = 0; t < kBlk; ++t) {
      double acc = t == c ? 1.0 : 0.0;
#pragma unroll
      for (int u = 0; u < t; ++u) acc = __builtin_fma(-Gs[b0 + t][b0 + u], x[u], acc);
      x[t] = acc / Gs[b0 + t][b0 + t];
    }
#pragma unroll
    for (int t = 0; t < kBlk; ++t) Dinv[(b0 + t) * kBlk + c] = x[t];
  }
  if (tid == 0) {
    const int32_t prev = reset ? 0 : *flag;
    *flag = prev | bad;
  }
}

// Row-wise triangular solves with the factor C (lower, kR x kR, zero past r)
// of the last small_cholesky_kernel, blocked by 16 columns on the float64
// matrix cores (MFMA 16x16x4: A element (row l%16, k l/16), B element
// (k l/16, column l%16), accumulator register q of lane l at row l/16 + 4q,
// column l%16).  Each wave owns 16 rows:
//   Z = Y C^{-T}:  Z_b = (Y_b - sum_{c<b} Z_c C_bc^T) D_b^T   (b = 0 .. 3)
//   K = Z C^{-1}:  K_b = (Z_b - sum_{c>b} K_c C_cb) D_b       (b = 3 .. 0)
// with D_b the inverse of diagonal block b.  Results go through the wave's
// LDS tiles to become A operands of the later blocks.  Columns past r are 0
// (Y is 0 there, C's blocks are 0 and D_b is the identity).
// WITH_K = false writes Z (n x r) to Out; WITH_K = true writes Z transposed
// (r x n) to Zt and K (n x r) to Out.
template <bool WITH_K>
__global__ __launch_bounds__(kThreads) void solve_rows_kernel(const double* __restrict__ C,
                                                              const double* __restrict__ Dinv,
                                                              const double* __restrict__ Y, int64_t n, int r,
                                                              double* __restrict__ Out, double* __restrict__ Zt) {
  __shared__ double W[kThreads / 64][kNBlk + 1][kBlk][kBlk + 1];   // per wave: 4 result blocks + staging
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 64 + 16 * wave;
  double (*T)[kBlk + 1] = W[wave][kNBlk];
  const doublex4 zero4 = {0.0, 0.0, 0.0, 0.0};

#pragma unroll
  for (int b = 0; b < kNBlk; ++b) {
    doublex4 acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = i0 + lq + 4 * q;
      const int col = kBlk * b + lr;
      acc[q] = (row < n && col < r) ? Y[row * r + col] : 0.0;
    }
#pragma unroll
    for (int c = 0; c < b; ++c)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const double av = -W[wave][c][lr][4 * s4 + lq];
        const double bv = C[(kBlk * b + lr) * kR + kBlk * c + 4 * s4 + lq];
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
      }
#pragma unroll
    for (int q = 0; q < 4; ++q) T[lq + 4 * q][lr] = acc[q];
    __syncthreads();
    doublex4 z = zero4;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      z = __builtin_amdgcn_mfma_f64_16x16x4f64(T[lr][4 * s4 + lq], Dinv[(kBlk * b + lr) * kBlk + 4 * s4 + lq], z,
                                              0, 0, 0);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) W[wave][b][lq + 4 * q][lr] = z[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = i0 + lq + 4 * q;
      const int col = kBlk * b + lr;
      if (row < n && col < r) {
        if (WITH_K) Zt[col * n + row] = z[q];
        else Out[row * r + col] = z[q];
      }
    }
  }
  if (!WITH_K) return;
#pragma unroll
  for (int b = kNBlk - 1; b >= 0; --b) {
    doublex4 acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = W[wave][b][lq + 4 * q][lr];
#pragma unroll
    for (int c = b + 1; c < kNBlk; ++c)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const double av = -W[wave][c][lr][4 * s4 + lq];
        const double bv = C[(kBlk * c + 4 * s4 + lq) * kR + kBlk * b + lr];
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
      }
#pragma unroll
    for (int q = 0; q < 4; ++q) T[lq + 4 * q][lr] = acc[q];
    __syncthreads();
    doublex4 k = zero4;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      k = __builtin_amdgcn_mfma_f64_16x16x4f64(T[lr][4 * s4 + lq], Dinv[(kBlk * b + 4 * s4 + lq) * kBlk + lr], k,
                                              0, 0, 0);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) W[wave][b][lq + 4 * q][lr] = k[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = i0 + lq + 4 * q;
      const int col = kBlk * b + lr;
      if (row < n && col < r) Out[row * r + col] = k[q];
    }
  }
}

// H_L[i][j] = (float)(H[i][j] - sum_a Z[i][a] Z[j][a]) on the matrix cores.
// Only tiles on or above the diagonal are computed; each off-diagonal tile is
// also written mirrored, so H_L is exactly symmetric (H must be symmetric: the
// upper tiles of H are read).  Four waves of 32 x 32 per 64 x 64 tile, K = r
// in STEPS 4-deep MFMA steps, operands read coalesced from Z transposed
// (Zt, r x n, L2-resident); the tile goes through LDS for coalesced row and
// column stores.
template <int STEPS>
__global__ __launch_bounds__(kThreads) void downdate_kernel(const float* __restrict__ H, int64_t ldh,
                                                            const double* __restrict__ Zt, int64_t n, int r,
                                                            float* __restrict__ HL, int64_t ldhl, int tiles) {
  __shared__ float T[kTP][kTP + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kl = lane >> 4, cl = lane & 15;
  int t = static_cast<int>(blockIdx.x), bi = 0;
  while (t >= tiles - bi) {
    t -= tiles - bi;
    ++bi;
  }
  const int bj = bi + t;
  const int64_t i0 = static_cast<int64_t>(bi) * kTP, j0 = static_cast<int64_t>(bj) * kTP;
  const int wr = wave >> 1, wc = wave & 1;
  double a[STEPS][2], b[STEPS][2];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int k = 4 * s + kl;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t i = i0 + 32 * wr + 16 * u + cl, j = j0 + 32 * wc + 16 * u + cl;
      a[s][u] = (k < r && i < n) ? Zt[k * n + i] : 0.0;
      b[s][u] = (k < r && j < n) ? Zt[k * n + j] : 0.0;
    }
  }
  doublex4 acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[u][v] = doublex4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 2; ++v) acc[u][v] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s][u], b[s][v], acc[u][v], 0, 0, 0);
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 32 * wr + 16 * u + kl + 4 * q, col = 32 * wc + 16 * v + cl;
        const int64_t i = i0 + row, j = j0 + col;
        const double h = (i < n && j < n) ? static_cast<double>(H[i * ldh + j]) : 0.0;
        T[row][col] = static_cast<float>(h - acc[u][v][q]);
      }
  __syncthreads();
  for (int e = tid; e < kTP * kTP; e += kThreads) {
    const int row = e / kTP, col = e % kTP;
    const int64_t i = i0 + row, j = j0 + col;
    if (i < n && j < n) HL[i * ldhl + j] = T[row][col];
    if (bi != bj) {
      const int64_t i2 = j0 + row, j2 = i0 + col;
      if (i2 < n && j2 < n) HL[i2 * ldhl + j2] = T[col][row];
    }
  }
}

// ---------------------------------------------------------------------------
// Fixed-grid refinement of the codes (Daily Papers page, GPTQ-intrinsic LoRA
// abstract: "Bid-Up", a refinement on the fixed grid that alternates with the
// optimal low-rank compensation and never increases the layer-wise error; no
// algorithm is printed).  Reading: cyclic coordinate descent.  Row i's error
// is 1/2 d H d^T with d = W_i - C_i - W^_i (C = (L R)^T held fixed, H the
// undamped H = 2 X^T X); moving column j's value by delta changes it by
// -delta g_j + delta^2 H_jj / 2, g = H d, so the best grid value of that
// column is the one nearest to W^_ij + g_j / H_jj, taken only when it lowers
// the error (H_jj = 0 columns do not take part).  Columns in original order.
//
// The residual is kept transposed, Dt[j][i] = d_i[j] (float64, n x m), so
// that one block's g for all rows is a tall product Dt^T H[:, block] on the
// float64 matrix cores (tall_mfma_kernel, split over K), and the in-block
// sequence runs one row per lane: per block of kRB columns, g from the
// product, then each column's decision and the update g_k -= delta H_jk of
// the block's later columns (the product of the next block sees every move
// made so far).  In exact arithmetic this is the column-by-column sequence.
// Float64 throughout; the decision arithmetic (v, rint, the gain) is written
// without contraction, in the order the definition gives it.
// ---------------------------------------------------------------------------
constexpr int kRB = 64;   // columns per refinement block (= kR, the product's column tile)
static_assert(kRB == kR, "one block is one column tile of the tall product");

// Dt[j][i] = (W[i][j] - sum_a R[a][i] L[j][a]) - s_g(j) (c - z_g(j)) for a
// 64 x 64 tile of (rows i, columns j); lane = row, wave = 16 columns.
template <int DT>
__global__ __launch_bounds__(kThreads) void refine_residual_kernel(
    const void* __restrict__ W, int64_t ldw, int64_t m, int64_t n, const double* __restrict__ L,
    const float* __restrict__ R, int r, int64_t ldr, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t G, int64_t group,
    const int32_t* __restrict__ gidx, double* __restrict__ Dt) {
  __shared__ double Ls[64][kR + 1];
  __shared__ double Rs[kR][64];
  const int tid = threadIdx.x, li = tid & 63, jg = tid >> 6;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 64, j0 = static_cast<int64_t>(blockIdx.y) * 64;
  for (int e = tid; e < 64 * r; e += kThreads) {
    const int jj = e / r, a = e % r;
    Ls[jj][a] = j0 + jj < n ? L[(j0 + jj) * r + a] : 0.0;
  }
  for (int e = tid; e < 64 * r; e += kThreads) {
    const int a = e >> 6, ii = e & 63;
    Rs[a][ii] = i0 + ii < m ? static_cast<double>(R[a * ldr + i0 + ii]) : 0.0;
  }
  __syncthreads();
  const int64_t i = i0 + li;
  if (i >= m) return;
  for (int jj = 16 * jg; jj < 16 * jg + 16; ++jj) {
    const int64_t j = j0 + jj;
    if (j >= n) break;
    double corr = 0.0;
    for (int a = 0; a < r; ++a) corr = __builtin_fma(Rs[a][li], Ls[jj][a], corr);
    const int64_t g = gidx ? static_cast<int64_t>(gidx[j]) : (group ? j / group : 0);
    const double s = static_cast<double>(scales[i * G + g]);
    const double z = static_cast<double>(zeros[i * G + g]);
    const double c = static_cast<double>(codes[i * n + j]);
    Dt[j * m + i] = (w_elem<DT>(W, i * ldw + j) - corr) - s * (c - z);
  }
}

__global__ void refine_clear_kernel(unsigned long long* __restrict__ p, int count) {
  const int e = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
  if (e < count) p[e] = 0ull;
}

// Block c0 .. c0+bw-1 for 64 rows (one wave; lane = row).  part holds the
// block's split partials of Dt^T H[:, block] (kR columns per row, zero past
// bw).  Writes the block's codes and residual columns; adds the number of
// moves to *count (when not null).
//
// The block's diagonal block of H (widened to float64), each row's grid and
// each row's gradient entries are staged in LDS (lane = row: gl[k][lane]),
// so the column walk reads no global memory.  Columns go in sub-blocks of
// kRSub: the sub-block's gradient entries are held in registers; a column's
// decision is followed at once by the corrections of the sub-block's later
// columns, and the block's columns after the sub-block take the sub-block's
// corrections in one pass at its end.  For every column k the corrections
// still arrive in increasing j, each as g_k = g_k - delta_j H_kj, so this is
// the column-by-column sequence with the loop over k reordered only.
constexpr int kRSub = 8;
static_assert(kRSub == 8 && kRB % kRSub == 0, "whole sub-blocks of eight columns");

template <bool FULL>
__global__ __launch_bounds__(64) void refine_sweep_kernel(
    const double* __restrict__ part, int splits, int64_t m, int64_t n, int c0, int bw_arg,
    const float* __restrict__ H, int64_t ldh, const float* __restrict__ scales, const uint8_t* __restrict__ zeros,
    int64_t G, int64_t group, const int32_t* __restrict__ gidx, double maxq, int codes_vec,
    uint8_t* __restrict__ codes, double* __restrict__ Dt, unsigned long long* __restrict__ count) {
#pragma clang fp contract(off)
  const int bw = FULL ? kRB : bw_arg;   // a whole block: every column test below is decided at compile time
  __shared__ float2 grid[kRB][64];                              // (s, z) of each column for each lane's row
  __shared__ __attribute__((aligned(16))) double hs[kRB][kRB];  // H[c0 + r][c0 + c] widened, zero past bw
  __shared__ double gl[kRB][64];                                // gradient entry k of each lane's row
  __shared__ int gcol[kRB];                                     // group of each column
  const int lane = static_cast<int>(threadIdx.x);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const bool active = i < m;
  const int64_t ir = active ? i : m - 1;   // lanes past m follow row m-1 and write nothing
  const float* hb = H + static_cast<int64_t>(c0) * ldh + c0;
  // Every load that does not depend on another goes out first: column l of
  // the H block, the group of column l, this row's codes, the first split's
  // partials; then they are consumed.
  float hv[kRB];
#pragma unroll
  for (int r = 0; r < kRB; ++r) hv[r] = (r < bw && lane < bw) ? hb[static_cast<int64_t>(r) * ldh + lane] : 0.f;
  const int64_t col_l = c0 + lane;
  const int gc = lane < bw ? (gidx ? static_cast<int>(gidx[col_l]) : (group ? static_cast<int>(col_l / group) : 0)) : 0;
  uint32_t cw[kRB / 4];
  uint8_t* crow = codes + ir * n + c0;
  if (codes_vec && bw == kRB) {
#pragma unroll
    for (int q = 0; q < kRB / 16; ++q) {
      const u32x4 v = reinterpret_cast<const u32x4*>(crow)[q];
      cw[4 * q] = v[0]; cw[4 * q + 1] = v[1]; cw[4 * q + 2] = v[2]; cw[4 * q + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int q = 0; q < kRB / 4; ++q) {
      uint32_t v = 0u;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (4 * q + t < bw) v |= static_cast<uint32_t>(crow[4 * q + t]) << (8 * t);
      cw[q] = v;
    }
  }
  // The gradient entries: the split partials summed in split order into
  // gl (0 + p_0 + p_1 + ...), one round trip per split.
  for (int t = 0; t < splits; ++t) {
    const doublex4* pp = reinterpret_cast<const doublex4*>(part + (static_cast<int64_t>(t) * m + ir) * kR);
    doublex4 pv[kRB / 4];
#pragma unroll
    for (int v = 0; v < kRB / 4; ++v) pv[v] = pp[v];
    if (t == 0) {
      gcol[lane] = gc;
#pragma unroll
      for (int r = 0; r < kRB; ++r) hs[r][lane] = static_cast<double>(hv[r]);
    }
#pragma unroll
    for (int v = 0; v < kRB / 4; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) gl[4 * v + e][lane] = (t == 0 ? 0.0 : gl[4 * v + e][lane]) + pv[v][e];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kRB; ++j) {
    if (j < bw) {
      const int64_t gg = gcol[j];
      grid[j][lane] = float2{scales[ir * G + gg], static_cast<float>(zeros[ir * G + gg])};
    }
  }
  __syncthreads();

  int moved = 0;
  // Every index into g, dl and cw is a compile-time constant after unrolling
  // (bw is a uniform guard, not a trip count), so they stay in registers.
#pragma unroll
  for (int sb = 0; sb < kRB; sb += kRSub) {
    // The sub-block's gradient entries, grid values and H triangle (H_kj
    // for sb <= j <= k < sb + kRSub) go to registers in one batch.
    double g[kRSub], dl[kRSub], ht[kRSub * (kRSub + 1) / 2];
    float2 sz[kRSub];
#pragma unroll
    for (int jj = 0; jj < kRSub; ++jj) {
      g[jj] = gl[sb + jj][lane];
      sz[jj] = grid[sb + jj][lane];
    }
#pragma unroll
    for (int kk = 0; kk < kRSub; ++kk)
#pragma unroll
      for (int jj = 0; jj <= kk; ++jj) ht[kk * (kk + 1) / 2 + jj] = hs[sb + kk][sb + jj];
    // Branch-free decisions: every lane evaluates the candidate code, its
    // step and its gain, and takes the step only if the walk would (a
    // column past bw, a dead column, no change or no gain keeps the code).
    // A step not taken is zero; subtracting zero times H leaves every
    // gradient entry unchanged (up to the sign of a zero, which no decision
    // depends on).
#pragma unroll
    for (int jj = 0; jj < kRSub; ++jj) {
      const int j = sb + jj;
      const double hjj = ht[jj * (jj + 1) / 2 + jj];
      const double s = static_cast<double>(sz[jj].x), z = static_cast<double>(sz[jj].y);
      const int sh = 8 * (j & 3);
      const int cold = static_cast<int>((cw[j >> 2] >> sh) & 0xffu);
      const double what = s * (static_cast<double>(cold) - z);
      const double v = what + g[jj] / hjj;
      const double q = fmin(fmax(rint(v / s) + z, 0.0), maxq);
      const int cn = static_cast<int>(q);
      const double d = s * (static_cast<double>(cn) - z) - what;
      const double gain = d * g[jj] - 0.5 * d * d * hjj;
      const bool take = j < bw && active && hjj > 0.0 && cn != cold && gain > 0.0;
      const double delta = take ? d : 0.0;
      cw[j >> 2] = take ? ((cw[j >> 2] & ~(0xffu << sh)) | (static_cast<uint32_t>(cn) << sh)) : cw[j >> 2];
      moved += take ? 1 : 0;
      dl[jj] = delta;
      // the sub-block's later columns (H past bw is zero; g there is unused)
#pragma unroll
      for (int kk = jj + 1; kk < kRSub; ++kk) g[kk] = g[kk] - delta * ht[kk * (kk + 1) / 2 + jj];
    }
    // The block's columns after the sub-block, eight at a time: H[k][sb ..
    // sb+7] is one contiguous row piece (H_jk = H_kj, H being exactly
    // symmetric).  All reads of a group are issued before its arithmetic.
    for (int k0 = sb + kRSub; k0 < kRB; k0 += 8) {
      doublex4 h0[8], h1[8];
      double gk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        h0[u] = *reinterpret_cast<const doublex4*>(&hs[k0 + u][sb]);
        h1[u] = *reinterpret_cast<const doublex4*>(&hs[k0 + u][sb + 4]);
        gk[u] = gl[k0 + u][lane];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int u = 0; u < 8; ++u) gk[u] = gk[u] - dl[e] * h0[u][e];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int u = 0; u < 8; ++u) gk[u] = gk[u] - dl[4 + e] * h1[u][e];
#pragma unroll
      for (int u = 0; u < 8; ++u) gl[k0 + u][lane] = gk[u];
    }
  }

  if (active) {
    // codes and the residual of each moved column: d_j -= delta, delta
    // recomputed from the old and new codes exactly as in the walk
    uint32_t c_old[kRB / 4];
    if (codes_vec && bw == kRB) {
#pragma unroll
      for (int q = 0; q < kRB / 16; ++q) {
        const u32x4 v = reinterpret_cast<const u32x4*>(crow)[q];
        c_old[4 * q] = v[0]; c_old[4 * q + 1] = v[1]; c_old[4 * q + 2] = v[2]; c_old[4 * q + 3] = v[3];
      }
#pragma unroll
      for (int q = 0; q < kRB / 16; ++q)
        reinterpret_cast<u32x4*>(crow)[q] = u32x4{cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]};
    } else {
#pragma unroll
      for (int q = 0; q < kRB / 4; ++q) {
        uint32_t v = 0u;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (4 * q + t < bw) v |= static_cast<uint32_t>(crow[4 * q + t]) << (8 * t);
        c_old[q] = v;
      }
      for (int j = 0; j < bw; ++j) crow[j] = static_cast<uint8_t>(cw[j >> 2] >> (8 * (j & 3)));
    }
    // The residual entries of the block are read in one batch before any is
    // written (one round trip instead of one per column: the compiler
    // cannot tell the columns' addresses apart).
    double* drow = Dt + static_cast<int64_t>(c0) * m + i;
#pragma unroll
    for (int h = 0; h < kRB; h += 32) {
      double dold[32];
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) dold[jj] = h + jj < bw ? drow[static_cast<int64_t>(h + jj) * m] : 0.0;
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) {
        const int j = h + jj;
        if (j >= bw) continue;
        const int co = static_cast<int>((c_old[j >> 2] >> (8 * (j & 3))) & 0xffu);
        const int cn = static_cast<int>((cw[j >> 2] >> (8 * (j & 3))) & 0xffu);
        if (co != cn) {
          const float2 sz = grid[j][lane];
          const double s = static_cast<double>(sz.x), z = static_cast<double>(sz.y);
          const double d = s * (static_cast<double>(cn) - z) - s * (static_cast<double>(co) - z);
          drow[static_cast<int64_t>(j) * m] = dold[jj] - d;
        }
      }
    }
  }
  if (count != nullptr) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) moved += __shfl_xor(moved, off);
    if (lane == 0 && moved > 0) atomicAdd(count, static_cast<unsigned long long>(moved));
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
  int64_t want = ceil_div(kCompensationBlocks, s.tiles);
  const int64_t cap = std::max<int64_t>(1, stages / 4);
  want = std::max<int64_t>(1, std::min(want, cap));
  s.kchunk = ceil_div(stages, want) * kTK;
  s.splits = ceil_div(K, s.kchunk);
  return s;
}

// Splits of the matrix-core product: K in multiples of kMChunk, enough
// workgroups of kMP rows to cover the chip twice over.
Split choose_split_mfma(int64_t P, int64_t K, int64_t max_splits, int64_t target_blocks = kTargetBlocks) {
  Split s;
  s.tiles = ceil_div(P, kMP);
  const int64_t stages = ceil_div(K, kMChunk);
  const int64_t want =
      std::max<int64_t>(1, std::min({ceil_div(target_blocks, s.tiles), stages, max_splits}));
  s.kchunk = ceil_div(stages, want) * kMChunk;
  s.splits = ceil_div(K, s.kchunk);
  return s;
}

size_t part_bytes(const Split& s, int64_t P) {
  return static_cast<size_t>(s.splits) * static_cast<size_t>(P) * kR * sizeof(double);
}

struct Layout {
  size_t off_part, off_y, off_q, off_g, off_c, off_dinv, off_flag, total;
};

Layout lowrank_layout(int64_t m, int64_t n, int64_t r) {
  Layout L;
  size_t part = std::max(part_bytes(choose_split_mfma(n, n, kTargetBlocks), n),
                         part_bytes(choose_split_mfma(r, n, kMaxGramSplits), r));
  if (m > 0) part = std::max(part, part_bytes(choose_split(m, n), m));
  const size_t nr = static_cast<size_t>(n) * static_cast<size_t>(r) * sizeof(double);
  L.off_part = 0;
  L.off_y = align256(part);
  L.off_q = align256(L.off_y + nr);
  L.off_g = align256(L.off_q + nr);
  L.off_c = align256(L.off_g + kR * kR * sizeof(double));
  L.off_dinv = align256(L.off_c + kR * kR * sizeof(double));
  L.off_flag = align256(L.off_dinv + kR * kBlk * sizeof(double));
  L.total = align256(L.off_flag + sizeof(int32_t));
  return L;
}

struct Ctx {
  hipStream_t st;
  double* part;
  double* Y;
  double* Q;
  double* G;
  double* C;
  double* dinv;
  int32_t* flag;
};

Ctx make_ctx(const Layout& L, void* ws, void* stream) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  Ctx c;
  c.st = static_cast<hipStream_t>(stream);
  c.part = reinterpret_cast<double*>(base + L.off_part);
  c.Y = reinterpret_cast<double*>(base + L.off_y);
  c.Q = reinterpret_cast<double*>(base + L.off_q);
  c.G = reinterpret_cast<double*>(base + L.off_g);
  c.C = reinterpret_cast<double*>(base + L.off_c);
  c.dinv = reinterpret_cast<double*>(base + L.off_dinv);
  c.flag = reinterpret_cast<int32_t*>(base + L.off_flag);
  return c;
}

template <int DT>
gptq_status launch_compensation(TallArgs a, const Ctx& c, Split* used) {
  const Split s = choose_split(a.P, a.K);
  a.kchunk = s.kchunk;
  a.part = c.part;
  compensation_kernel<DT><<<dim3(static_cast<unsigned>(s.tiles), static_cast<unsigned>(s.splits)), kThreads, 0,
                            c.st>>>(a);
  GPTQ_TRY_LAUNCH();
  *used = s;
  return GPTQ_OK;
}

// part = the split partials of S^T B for S K x P (float32 or float64,
// leading dimension lds) and B K x r.
template <typename ST>
Split partial_t(const ST* S, int64_t lds, const double* B, int64_t P, int64_t K, int64_t r, int64_t max_splits,
                const Ctx& c) {
  const Split s = choose_split_mfma(P, K, max_splits);
  tall_mfma_kernel<ST><<<dim3(static_cast<unsigned>(s.tiles), static_cast<unsigned>(s.splits)), kThreads, 0,
                         c.st>>>(S, lds, B, r, P, K, static_cast<int>(r), s.kchunk, c.part);
  return s;
}

// Out (n x r, float64) = H X for X n x r (H symmetric: A(p, k) = H[k][p]).
gptq_status product_h(const float* H, int64_t ldh, const double* X, int64_t n, int64_t r, double* Out,
                      const Ctx& c) {
  const Split s = partial_t<float>(H, ldh, X, n, n, r, kTargetBlocks, c);
  GPTQ_TRY_LAUNCH();
  reduce_splits_kernel<false><<<static_cast<unsigned>(ceil_div(n * r, kThreads)), kThreads, 0, c.st>>>(
      c.part, static_cast<int>(s.splits), n, r, Out, r);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

// C (and 1 / diag C) from the Cholesky factor of A^T B (A, B n x r).
gptq_status factor_gram(const double* A, const double* B, int64_t n, int64_t r, const Ctx& c, int reset) {
  const Split s = partial_t<double>(A, r, B, r, n, r, kMaxGramSplits, c);
  GPTQ_TRY_LAUNCH();
  reduce_splits_kernel<false><<<static_cast<unsigned>(ceil_div(r * r, kThreads)), kThreads, 0, c.st>>>(
      c.part, static_cast<int>(s.splits), r, r, c.G, r);
  GPTQ_TRY_LAUNCH();
  small_cholesky_kernel<<<1, kThreads, 0, c.st>>>(c.G, static_cast<int>(r), c.C, c.dinv, c.flag, reset);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

// Out = Y C^{-T} with C C^T = Y^T Y: orthonormal columns spanning Y's.
gptq_status orthonormalize(const double* Y, int64_t n, int64_t r, double* Out, const Ctx& c, int reset) {
  gptq_status rc = factor_gram(Y, Y, n, r, c, reset);
  if (rc != GPTQ_OK) return rc;
  solve_rows_kernel<false><<<static_cast<unsigned>(ceil_div(n, 64)), kThreads, 0, c.st>>>(
      c.C, c.dinv, Y, n, static_cast<int>(r), Out, nullptr);
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

// Refinement workspace: the transposed residual Dt (n x m float64) and the
// split partials of one block's product.
struct RefineLayout {
  Split split;
  size_t off_dt, off_part, total;
};

RefineLayout refine_layout(int64_t m, int64_t n) {
  RefineLayout L;
  // three workgroups per CU (the product's registers and LDS allow three)
  L.split = choose_split_mfma(m, n, kRefineBlocks, kRefineBlocks);
  L.off_dt = 0;
  L.off_part = align256(static_cast<size_t>(n) * static_cast<size_t>(m) * sizeof(double));
  L.total = align256(L.off_part + part_bytes(L.split, m));
  return L;
}

template <int DT>
gptq_status launch_refine_residual(const void* W, int64_t ldw, int64_t m, int64_t n, const double* L,
                                   const float* R, int64_t r, int64_t ldr, const uint8_t* codes,
                                   const float* scales, const uint8_t* zeros, int64_t G, int64_t group,
                                   const int32_t* gidx, double* Dt, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ceil_div(m, 64)), static_cast<unsigned>(ceil_div(n, 64)));
  refine_residual_kernel<DT><<<grid, kThreads, 0, st>>>(W, ldw, m, n, L, R, static_cast<int>(r), ldr, codes, scales,
                                                        zeros, G, group, gidx, Dt);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

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
  solve_rows_kernel<true><<<static_cast<unsigned>(ceil_div(n, 64)), kThreads, 0, c.st>>>(
      c.C, c.dinv, c.Y, n, static_cast<int>(r), K, c.Q);                 // Zt = (Y C^{-T})^T, K = Z C^{-1}
  GPTQ_TRY_LAUNCH();
  const int t = static_cast<int>(ceil_div(n, kTP));
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(t) * (t + 1) / 2);
  const int ri = static_cast<int>(r);
  if (r <= 8) downdate_kernel<2><<<blocks, kThreads, 0, c.st>>>(H, ldh, c.Q, n, ri, H_L, ldhl, t);
  else if (r <= 16) downdate_kernel<4><<<blocks, kThreads, 0, c.st>>>(H, ldh, c.Q, n, ri, H_L, ldhl, t);
  else if (r <= 32) downdate_kernel<8><<<blocks, kThreads, 0, c.st>>>(H, ldh, c.Q, n, ri, H_L, ldhl, t);
  else downdate_kernel<16><<<blocks, kThreads, 0, c.st>>>(H, ldh, c.Q, n, ri, H_L, ldhl, t);
  GPTQ_TRY_LAUNCH();
  return read_flag(c);
}

extern "C" gptq_status gptq_lowrank_compensation(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw,
                                                 const uint8_t* codes, const float* scales, const uint8_t* zeros,
                                                 int group_size, const int32_t* g_idx, const double* K, int64_t r,
                                                 float* R, int64_t ldr, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !codes || !scales || !zeros || !K || !R || !valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (m < 1 || !rank_ok(n, r) || ldw < n || ldr < m || group_size < 0) return GPTQ_ERR_INVALID_ARG;
  const Layout lay = lowrank_layout(m, n, r);
  if (!ws || ws_bytes < lay.total) return GPTQ_ERR_WORKSPACE;
  const Ctx c = make_ctx(lay, ws, stream);
  TallArgs a = {};
  a.A = W; a.lda = ldw; a.codes = codes; a.scales = scales; a.zeros = zeros;
  a.group = group_size; a.G = group_size ? ceil_div(n, group_size) : 1; a.gidx = g_idx;
  a.B = K; a.ldb = r; a.P = m; a.K = n; a.r = r;
  Split s;
  gptq_status rc = w_dtype == GPTQ_F32  ? launch_compensation<GPTQ_F32>(a, c, &s)
                   : w_dtype == GPTQ_F16 ? launch_compensation<GPTQ_F16>(a, c, &s)
                                         : launch_compensation<GPTQ_BF16>(a, c, &s);
  if (rc != GPTQ_OK) return rc;
  reduce_splits_kernel<true><<<static_cast<unsigned>(ceil_div(m * r, kThreads)), kThreads, 0, c.st>>>(
      c.part, static_cast<int>(s.splits), m, r, R, ldr);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

// Sizes the refinement takes: rows and columns each below 2^31, at most 2^48
// residual entries.
static bool refine_size_ok(int64_t m, int64_t n) {
  return m >= 1 && n >= 1 && m <= INT32_MAX && n <= INT32_MAX && m <= ((int64_t)1 << 48) / n;
}

extern "C" size_t gptq_refine_ws_bytes(int64_t m, int64_t n) {
  if (!refine_size_ok(m, n)) return 0;
  return refine_layout(m, n).total;
}

extern "C" gptq_status gptq_refine_codes(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw,
                                         const float* H, int64_t ldh, const double* L, const float* R, int64_t r,
                                         int64_t ldr, const float* scales, const uint8_t* zeros, int group_size,
                                         const int32_t* g_idx, int levels, int sweeps, uint8_t* codes,
                                         int64_t* moves, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !H || !scales || !zeros || !codes || !valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (!refine_size_ok(m, n) || ldw < n || ldh < n) return GPTQ_ERR_INVALID_ARG;
  if (levels < 2 || levels > 256 || sweeps < 0 || group_size < 0) return GPTQ_ERR_INVALID_ARG;
  if (r < 0 || r > kR || r > n) return GPTQ_ERR_INVALID_ARG;
  if (r > 0 && (!L || !R || ldr < m)) return GPTQ_ERR_INVALID_ARG;
  const RefineLayout lay = refine_layout(m, n);
  if (!ws || ws_bytes < lay.total) return GPTQ_ERR_WORKSPACE;
  if (sweeps == 0) return GPTQ_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned char* base = static_cast<unsigned char*>(ws);
  double* Dt = reinterpret_cast<double*>(base + lay.off_dt);
  double* part = reinterpret_cast<double*>(base + lay.off_part);
  const int64_t G = group_size ? ceil_div(n, group_size) : 1;
  gptq_status rc = w_dtype == GPTQ_F32
                       ? launch_refine_residual<GPTQ_F32>(W, ldw, m, n, L, R, r, ldr, codes, scales, zeros, G,
                                                          group_size, g_idx, Dt, st)
                   : w_dtype == GPTQ_F16
                       ? launch_refine_residual<GPTQ_F16>(W, ldw, m, n, L, R, r, ldr, codes, scales, zeros, G,
                                                          group_size, g_idx, Dt, st)
                       : launch_refine_residual<GPTQ_BF16>(W, ldw, m, n, L, R, r, ldr, codes, scales, zeros, G,
                                                           group_size, g_idx, Dt, st);
  if (rc != GPTQ_OK) return rc;
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(moves);
  if (cnt != nullptr) {
    refine_clear_kernel<<<static_cast<unsigned>(ceil_div(sweeps, 256)), 256, 0, st>>>(cnt, sweeps);
    GPTQ_TRY_LAUNCH();
  }
  const int codes_vec = (reinterpret_cast<uintptr_t>(codes) & 15) == 0 && n % 16 == 0;
  const Split& sp = lay.split;
  const int nblk = static_cast<int>(ceil_div(n, kRB));
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int b = 0; b < nblk; ++b) {
      const int c0 = b * kRB;
      const int bw = static_cast<int>(std::min<int64_t>(kRB, n - c0));
      tall_mfma_kernel<double, float>
          <<<dim3(static_cast<unsigned>(sp.tiles), static_cast<unsigned>(sp.splits)), kThreads, 0, st>>>(
              Dt, m, H + c0, ldh, m, n, bw, sp.kchunk, part);
      GPTQ_TRY_LAUNCH();
      if (bw == kRB)
        refine_sweep_kernel<true><<<static_cast<unsigned>(ceil_div(m, 64)), 64, 0, st>>>(
            part, static_cast<int>(sp.splits), m, n, c0, bw, H, ldh, scales, zeros, G, group_size, g_idx,
            static_cast<double>(levels - 1), codes_vec, codes, Dt, cnt ? cnt + sw : nullptr);
      else
        refine_sweep_kernel<false><<<static_cast<unsigned>(ceil_div(m, 64)), 64, 0, st>>>(
            part, static_cast<int>(sp.splits), m, n, c0, bw, H, ldh, scales, zeros, G, group_size, g_idx,
            static_cast<double>(levels - 1), codes_vec, codes, Dt, cnt ? cnt + sw : nullptr);
      GPTQ_TRY_LAUNCH();
    }
  }
  return GPTQ_OK;
}
