// Asymmetric calibration target (GPTAQ / GPTQv2 abstract, Daily Papers and
// mlsanity pages: the quantized layer's output on the quantized model's inputs
// Xq is matched to the full-precision output on the full-precision inputs
// Xf).  With W' = argmin_V ||Xq V^T - Xf W^T||^2 every Q has
// ||Xq Q^T - Xf W^T||^2 = ||Xq (Q - W')^T||^2 + const, so the objective is
// GPTQ's with H = 2 Xq^T Xq on the target W'.  With GPTQ's damping,
//   W' = W Hc^T H_d^{-1},  Hc = 2 Xq^T Xf,  H_d^{-1} = U^T U (processing order),
// computed as three float32 matrix products on the matrix cores:
//   G = W Hc^T,  Gp = G[:, perm],  T = Gp U^T,  Wp = T U,  W'[:, perm] = Wp,
// the two products with U skipping the K ranges where U is zero.
// Hc and H come from one gptq_hessian_accumulate call on [Xq | Xf].
#include "common.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;
constexpr int kTM = 128;  // C tile rows
constexpr int kTN = 128;  // C tile columns
constexpr int kTK = 32;   // K per stage

struct GemmLds {
  float As[2][kTM][kTK + 1];
  float Bs[2][kTK][kTN + 4];
};

template <int DT>
__device__ inline floatx4 load_a4(const void* A, int64_t off, bool vec, int valid) {
  floatx4 v = {0.f, 0.f, 0.f, 0.f};
  if (DT == GPTQ_F32 && vec && valid == 4) {
    v = *reinterpret_cast<const floatx4*>(static_cast<const float*>(A) + off);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < valid) v[t] = load_as_f32<DT>(A, off + t);
  }
  return v;
}

// C (M x N, row-major, ldc) = A (M x K, row-major, lda, element type DT) times
// B (K x N, row-major) or, with BT, B^T where B is N x K row-major.  float32
// MFMA 32x32x2, 128 x 128 tiles per workgroup (4 waves of 64 x 64), K staged
// 32 deep through two LDS buffers with the next stage loaded into registers
// while the current one multiplies.
// TRI = 1: B^T with B upper triangular (B[i][k] = 0 for k < i), so a column
// tile starting at col0 needs K from col0 on; TRI = 2: B upper triangular
// (B[k][j] = 0 for k > j), so a column tile needs K below col0 + kTN only.
template <int DT, bool BT, int TRI>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(const void* __restrict__ A, int64_t lda,
                                                            const float* __restrict__ B, int64_t ldb,
                                                            float* __restrict__ C, int64_t ldc, int M, int N,
                                                            int K) {
  __shared__ GemmLds L;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1;
  const int row0 = (int)blockIdx.y * kTM, col0 = (int)blockIdx.x * kTN;
  const bool veca = DT == GPTQ_F32 && (lda & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
  const bool vecb = (ldb & 3) == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  floatx16 acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = floatx16{};
  floatx4 ra[4], rb4[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + kThreads * i;
      const int r = e >> 3, k = (e & 7) * 4;
      const int row = row0 + r;
      const int valid = row < M ? max(0, min(4, K - (k0 + k))) : 0;
      ra[i] = load_a4<DT>(A, (int64_t)(row < M ? row : 0) * lda + k0 + k, veca, valid);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + kThreads * i;
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BT) {
        // B row (C column) c, K positions k .. k+3
        const int c = e >> 3, k = (e & 7) * 4;
        const int col = col0 + c;
        if (col < N) {
          const float* p = B + (int64_t)col * ldb + k0 + k;
          if (vecb && k0 + k + 4 <= K) {
            v = *reinterpret_cast<const floatx4*>(p);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = k0 + k + t < K ? p[t] : 0.f;
          }
        }
      } else {
        // B row (K position) kk, C columns c .. c+3
        const int kk = e >> 5, c = (e & 31) * 4;
        if (k0 + kk < K) {
          const float* p = B + (int64_t)(k0 + kk) * ldb + col0 + c;
          if (vecb && col0 + c + 4 <= N) {
            v = *reinterpret_cast<const floatx4*>(p);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = col0 + c + t < N ? p[t] : 0.f;
          }
        }
      }
      rb4[i] = v;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + kThreads * i;
      const int r = e >> 3, k = (e & 7) * 4;
#pragma unroll
      for (int t = 0; t < 4; ++t) L.As[buf][r][k + t] = ra[i][t];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + kThreads * i;
      if constexpr (BT) {
        const int c = e >> 3, k = (e & 7) * 4;
#pragma unroll
        for (int t = 0; t < 4; ++t) L.Bs[buf][k + t][c] = rb4[i][t];
      } else {
        const int kk = e >> 5, c = (e & 31) * 4;
        *reinterpret_cast<floatx4*>(&L.Bs[buf][kk][c]) = rb4[i];
      }
    }
  };
  const int k_lo = TRI == 1 ? col0 : 0;
  const int k_hi = TRI == 2 ? min(K, col0 + kTN) : K;
  const int nst = k_hi > k_lo ? (k_hi - k_lo + kTK - 1) / kTK : 0;
  if (nst > 0) {
    gload(k_lo);
    lstore(0);
  }
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    const bool next = s + 1 < nst;
    if (next) gload(k_lo + (s + 1) * kTK);
#pragma unroll
    for (int k2 = 0; k2 < kTK / 2; ++k2) {
      const int k = k2 * 2 + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) a[rb] = L.As[buf][wr * 64 + rb * 32 + (lane & 31)][k];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) b[cb] = L.Bs[buf][k][wc * 64 + cb * 32 + (lane & 31)];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
    }
    // Buffer buf ^ 1 was last read in stage s - 1, before the previous barrier.
    if (next) lstore(buf ^ 1);
    __syncthreads();
  }
  // 32x32 accumulator: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wr * 64 + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = col0 + wc * 64 + cb * 32 + (lane & 31);
        if (row < M && col < N) C[(int64_t)row * ldc + col] = acc[rb][cb][r];
      }
}

// out[r, j] = in[r, perm[j]] (gather) or out[r, perm[j]] = in[r, j] (scatter).
template <bool GATHER>
__global__ __launch_bounds__(kThreads) void permute_cols_kernel(const float* __restrict__ in, int64_t ldi,
                                                                const int32_t* __restrict__ perm, int n,
                                                                float* __restrict__ out, int64_t ldo) {
  const int64_t r = blockIdx.x;
  for (int j = threadIdx.x; j < n; j += kThreads) {
    if (GATHER)
      out[r * ldo + j] = in[r * ldi + perm[j]];
    else
      out[r * ldo + perm[j]] = in[r * ldi + j];
  }
}

template <int DT, bool BT, int TRI = 0>
void gemm(hipStream_t st, const void* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc, int M,
          int N, int K) {
  const dim3 grid((unsigned)ceil_div(N, kTN), (unsigned)ceil_div(M, kTM));
  gemm_f32_kernel<DT, BT, TRI><<<grid, kThreads, 0, st>>>(A, lda, B, ldb, C, ldc, M, N, K);
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_asym_target_ws_bytes(int64_t m, int64_t n) {
  if (m <= 0 || n <= 0) return 0;
  return 2 * align256((size_t)m * (size_t)n * sizeof(float));
}

extern "C" gptq_status gptq_asym_target(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw,
                                        const float* Hc, int64_t ldhc, const float* U, const int32_t* perm,
                                        float* Wt, int64_t ldwt, void* ws, size_t ws_bytes, void* stream) {
  if (m < 0 || n < 0 || !valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (m > ((int64_t)1 << 31) - 1 || n > ((int64_t)1 << 16)) return GPTQ_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return GPTQ_OK;
  if (W == nullptr || Hc == nullptr || U == nullptr || Wt == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (ldw < n || ldhc < n || ldwt < n) return GPTQ_ERR_INVALID_ARG;
  const size_t need = gptq_asym_target_ws_bytes(m, n);
  if (ws == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* b0 = static_cast<float*>(ws);
  float* b1 = reinterpret_cast<float*>(static_cast<char*>(ws) + need / 2);
  const int M = (int)m, N = (int)n;
  // G = W Hc^T (original column order)
  if (w_dtype == GPTQ_F32)
    gemm<GPTQ_F32, true>(st, W, ldw, Hc, ldhc, b0, n, M, N, N);
  else if (w_dtype == GPTQ_F16)
    gemm<GPTQ_F16, true>(st, W, ldw, Hc, ldhc, b0, n, M, N, N);
  else
    gemm<GPTQ_BF16, true>(st, W, ldw, Hc, ldhc, b0, n, M, N, N);
  GPTQ_TRY_LAUNCH();
  // Gp = G[:, perm] (processing order)
  const float* gp = b0;
  if (perm != nullptr) {
    permute_cols_kernel<true><<<(unsigned)m, kThreads, 0, st>>>(b0, n, perm, N, b1, n);
    GPTQ_TRY_LAUNCH();
    gp = b1;
  }
  // T = Gp U^T, then Wp = T U (H_d^{-1} = U^T U in processing order)
  float* tb = perm != nullptr ? b0 : b1;
  gemm<GPTQ_F32, true, 1>(st, gp, n, U, n, tb, n, M, N, N);
  GPTQ_TRY_LAUNCH();
  if (perm != nullptr) {
    float* wp = b1;
    gemm<GPTQ_F32, false, 2>(st, tb, n, U, n, wp, n, M, N, N);
    GPTQ_TRY_LAUNCH();
    permute_cols_kernel<false><<<(unsigned)m, kThreads, 0, st>>>(wp, n, perm, N, Wt, ldwt);
  } else {
    gemm<GPTQ_F32, false, 2>(st, tb, n, U, n, Wt, ldwt, M, N, N);
  }
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}
