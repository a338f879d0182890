// Stage 3: the GPTQ column sweep with lazy 128-column block updates.
// GPTQ knowledge note, "How It Works": after a column is quantized the
// columns still in full precision are adjusted with inverse-Hessian
// information; all rows follow one column order; 128-column blocks
// accumulate their corrections before a global update.  Wiki "GPTQ",
// "Technical Approach": low-bit grid with one scale per group.
//
// Rows are independent and run in parallel; columns are strictly sequential.
// For block kb (columns c0 .. c0+127 in processing order):
//   update_gemm   P = E[:, 0:c0] * U[0:c0, block]   (left-looking form of the
//                 deferred update; fp32 MFMA 32x32x2, split over K when there
//                 are too few row tiles to fill the GPU)
//   sweep         T = W[:, block] - sum(P); then 16-column sub-blocks: each
//                 row's 16 values are quantized in registers one column at a
//                 time (the error pushed into the sub-block's later columns
//                 with FMAs), and the sub-block's errors are pushed into the
//                 block's later columns with fp32 MFMA 16x16x4.
// The left-looking form applies each block's deferred corrections in one
// float32 accumulation (identical to the right-looking "update the rest after
// each block" form in exact arithmetic) and reads E instead of
// reading and rewriting the whole remaining weight matrix per block.
#include "common.h"

#include <type_traits>

namespace gptq {
namespace {

constexpr int kBS = 128;       // lazy block (columns)
constexpr int kSB = 16;        // register sub-block (columns)
constexpr int kRowsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kRowsPerWG = kRowsPerWave * kWaves;
constexpr int kThreads = 64 * kWaves;
static_assert(kThreads >= kBS, "one thread per column of the diagonal block");
constexpr int kTP = kBS + 4;   // LDS pitch of the block tile (floats)

// Grid parameters from a value range (float32, IEEE division, half-even).
__device__ inline void grid_from_range(float xmin, float xmax, float maxq, float& s, float& z,
                                       float& inv_s) {
  xmin = fminf(xmin, 0.f);
  xmax = fmaxf(xmax, 0.f);
  if (xmax == xmin) {
    xmin = -1.f;
    xmax = 1.f;
  }
  s = (xmax - xmin) / maxq;
  z = rintf((-xmin) / s);
  z = fminf(fmaxf(z, 0.f), maxq);
  inv_s = 1.f / s;
}

// c = clamp(rint(fl32(w / s)) + z, 0, maxq).  fl32(w / s) is obtained from
// the correctly rounded reciprocal inv_s = fl32(1/s) with one residual
// correction: q0 = fl32(w * inv_s), r = w - q0 * s (exact, fused),
// q = fl32(q0 + r * inv_s), which equals the correctly rounded quotient.
__device__ inline float quant_code(float w, float s, float inv_s, float z, float maxq) {
  const float q0 = w * inv_s;
  const float r = __builtin_fmaf(-q0, s, w);
  const float q = __builtin_fmaf(r, inv_s, q0);
  return fminf(fmaxf(rintf(q) + z, 0.f), maxq);
}

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}

// pinv[perm[j]] = j and g_idx[perm[j]] = j / g (0 when g = 0); identity
// when perm is NULL.  Out-of-range perm entries are clamped, never followed.
__global__ void index_kernel(int n, const int32_t* __restrict__ perm, int g, int32_t* __restrict__ pinv,
                             int32_t* __restrict__ gidx) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
    const int col = perm != nullptr ? min(max(perm[j], 0), n - 1) : j;
    if (pinv != nullptr) pinv[col] = j;
    if (gidx != nullptr) gidx[col] = g > 0 ? j / g : 0;
  }
}

// Rounds a float32 value to the storage type (round to nearest even).
template <int DT> __device__ inline void store_from_f32(void* p, int64_t i, float v);
template <> __device__ inline void store_from_f32<GPTQ_F32>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}
template <> __device__ inline void store_from_f32<GPTQ_F16>(void* p, int64_t i, float v) {
  // v is already rounded to float32; the empty asm keeps it so: without it
  // the compiler fuses a product feeding this conversion into one
  // v_fma_mixlo_f16, which rounds the exact product to float16 once and
  // differs from fl16(fl32(.)) where the float32 value lies on a float16 tie.
  asm volatile("" : "+v"(v));
  static_cast<_Float16*>(p)[i] = (_Float16)v;
}
template <> __device__ inline void store_from_f32<GPTQ_BF16>(void* p, int64_t i, float v) {
  const uint32_t u = __float_as_uint(v);
  static_cast<uint16_t*>(p)[i] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Row r of the sweep's codes (processing order) into original column order,
// in place (the row is staged in LDS first; pinv NULL: already in order), and
// the dequantized weights Wq[r][k] = fl_w(fl32(s_g (c - z_g))) of original
// column k, g = pinv[k] / group (Wq may be NULL).
template <int DT>
__global__ __launch_bounds__(256) void finalize_kernel(uint8_t* __restrict__ codes, int n,
                                                       const int32_t* __restrict__ pinv,
                                                       const float* __restrict__ scales,
                                                       const uint8_t* __restrict__ zeros, int g, int G,
                                                       void* __restrict__ Wq, int64_t ldq) {
  extern __shared__ __attribute__((aligned(16))) uint8_t row_s[];
  const int64_t r = blockIdx.x;
  uint8_t* row = codes + r * n;
  if (pinv != nullptr) {
    for (int j = threadIdx.x; j < n; j += 256) row_s[j] = row[j];
    __syncthreads();
  }
  for (int k = threadIdx.x; k < n; k += 256) {
    const int j = pinv != nullptr ? min(max(pinv[k], 0), n - 1) : k;
    const uint8_t c = pinv != nullptr ? row_s[j] : row[k];
    if (pinv != nullptr) row[k] = c;
    if (Wq != nullptr) {
      const int gi = g > 0 ? j / g : 0;
      const float sc = scales[r * G + gi];
      const float zc = (float)zeros[r * G + gi];
      store_from_f32<DT>(Wq, r * ldq + k, sc * ((float)c - zc));
    }
  }
}

// Four consecutive elements of W as float32; i is a multiple of 4 and the
// element address is 16-byte (float32) or 8-byte (16-bit types) aligned.
template <int DT> __device__ inline floatx4 load4_as_f32(const void* p, int64_t i);
template <> __device__ inline floatx4 load4_as_f32<GPTQ_F32>(const void* p, int64_t i) {
  return *reinterpret_cast<const floatx4*>(static_cast<const float*>(p) + i);
}
template <> __device__ inline floatx4 load4_as_f32<GPTQ_F16>(const void* p, int64_t i) {
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  const half4 h = *reinterpret_cast<const half4*>(static_cast<const _Float16*>(p) + i);
  return floatx4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
template <> __device__ inline floatx4 load4_as_f32<GPTQ_BF16>(const void* p, int64_t i) {
  const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
  return floatx4{__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u), __uint_as_float(b.y << 16),
                 __uint_as_float(b.y & 0xffff0000u)};
}

// Per-row grid (group_size 0): range of the original row, one wave per row.
template <int DT>
__global__ __launch_bounds__(256) void row_grid_kernel(const void* __restrict__ W, int64_t ldw, int m, int n,
                                                       float maxq, float* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= m) return;
  float mn = INFINITY, mx = -INFINITY;
  int j0 = 0;
  // Aligned rows: four elements per lane per load, four loads in flight.
  const int64_t align = DT == GPTQ_F32 ? 16 : 8;
  if ((reinterpret_cast<uintptr_t>(W) % align) == 0 && (ldw & 3) == 0) {
    const int n4 = n & ~3;
    for (; j0 + 4 * 4 * 64 <= n4; j0 += 4 * 4 * 64) {
      floatx4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = load4_as_f32<DT>(W, r * ldw + j0 + 4 * (lane + 64 * u));
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          mn = fminf(mn, v[u][k]);
          mx = fmaxf(mx, v[u][k]);
        }
    }
  }
  for (int j = j0 + lane; j < n; j += 64) {
    const float v = load_as_f32<DT>(W, r * ldw + j);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  if (lane == 0) {
    float s, z, inv_s;
    grid_from_range(mn, mx, maxq, s, z, inv_s);
    scales[r] = s;
    zeros[r] = (uint8_t)z;
  }
}

// P[sp][r][c] = sum_{k in split sp} E[r][k] * U[k][c0 + c]: a 128 x 128 tile
// per workgroup (4 waves of 64 x 64, fp32 MFMA 32x32x2).  K is staged 32 at a
// time through two LDS buffers: the next stage's E and U slabs are loaded
// into registers while the current stage is multiplied, then stored to the
// other buffer, with one barrier per stage.  A split covers whole stages.
constexpr int kUK = 32;          // K per stage
constexpr int kAP = kUK + 1;     // LDS pitch of the E slab (floats)

struct GemmLds {
  float As[2][128][kAP];
  __attribute__((aligned(16))) float Bs[2][kUK][kTP];
};

// Split sp of the row tile mt: K range [sp * stages_per_split * 32, ...)
// clipped to k_limit, for the columns of block kb.
__device__ __forceinline__ void update_gemm_body(const float* __restrict__ E, const float* __restrict__ U, int m,
                                                 int n, int kb, int k_limit, int stages_per_split,
                                                 float* __restrict__ P, int mt, int sp, GemmLds& L) {
  const int c0 = kb * kBS;
  const int bw = min(kBS, n - c0);
  const int k_begin = sp * stages_per_split * kUK;
  const int k_end = min(k_limit, k_begin + stages_per_split * kUK);
  const int row0 = mt * 128;
  const bool vec = (n & 3) == 0 && (reinterpret_cast<uintptr_t>(E) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(U) & 15) == 0;
  auto& As = L.As;
  auto& Bs = L.Bs;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1;
  floatx16 acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = floatx16{};

  // Stage slabs: E 128 x 32 and U 32 x 128, 1024 float4 each, 4 per thread.
  // Two register sets: the slabs of stage s + 2 are loaded while stage s is
  // multiplied and stage s + 1's (loaded a stage earlier) go to LDS, so each
  // HBM read of E has two stages of matrix-core work to arrive.
  floatx4 ea0[4], ub0[4], ea1[4], ub1[4];
  auto gload = [&](int k0, floatx4 (&ea)[4], floatx4 (&ub)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e >> 3, k = (e & 7) * 4;
      const int64_t row = row0 + r;
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
      if (row < m) {
        const float* p = E + row * n + k0 + k;
        if (vec) v = *reinterpret_cast<const floatx4*>(p);
        else v = floatx4{p[0], p[1], p[2], p[3]};
      }
      ea[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int kk = e >> 5, c = (e & 31) * 4;
      const float* p = U + (int64_t)(k0 + kk) * n + c0 + c;
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
      if (vec && c + 4 <= bw) {
        v = *reinterpret_cast<const floatx4*>(p);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (c + t < bw) ? p[t] : 0.f;
      }
      ub[i] = v;
    }
  };
  auto lstore = [&](int buf, const floatx4 (&ea)[4], const floatx4 (&ub)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e >> 3, k = (e & 7) * 4;
#pragma unroll
      for (int t = 0; t < 4; ++t) As[buf][r][k + t] = ea[i][t];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int kk = e >> 5, c = (e & 31) * 4;
      *reinterpret_cast<floatx4*>(&Bs[buf][kk][c]) = ub[i];
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int k2 = 0; k2 < kUK / 2; ++k2) {
      const int k = k2 * 2 + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) a[rb] = As[buf][wr * 64 + rb * 32 + (lane & 31)][k];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) b[cb] = Bs[buf][k][wc * 64 + cb * 32 + (lane & 31)];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
    }
  };

  const int nst = (k_end - k_begin) / kUK;
  if (nst > 0) {
    gload(k_begin, ea0, ub0);
    lstore(0, ea0, ub0);
  }
  if (nst > 1) gload(k_begin + kUK, ea1, ub1);
  __syncthreads();
  // Stage s is read from buffer s & 1.  A buffer is written only after the
  // barrier that follows its last read.
  for (int s = 0; s < nst; s += 2) {
    if (s + 2 < nst) gload(k_begin + (s + 2) * kUK, ea0, ub0);
    compute(0);
    if (s + 1 < nst) lstore(1, ea1, ub1);
    __syncthreads();
    if (s + 1 >= nst) break;
    if (s + 3 < nst) gload(k_begin + (s + 3) * kUK, ea1, ub1);
    compute(1);
    if (s + 2 < nst) lstore(0, ea0, ub0);
    __syncthreads();
  }
  // 32x32 accumulator: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + wr * 64 + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wc * 64 + cb * 32 + (lane & 31);
        if (row < m && col < bw) P[((int64_t)sp * m + row) * kBS + col] = acc[rb][cb][r];
      }
}

// Groups wider than one block (g a multiple of 128): at the group's first
// block c0 the range is taken over the current values of all its columns.
// For a later block b of the group those are W[:, b] - E[:, <c0] U[<c0, b];
// range_gemm_kernel forms the product's split partials (the deferred-update
// GEMM with its K range cut at c0) and range_reduce_kernel folds each row's
// min / max over block b into grange (first = 1 starts it afresh).
__global__ __launch_bounds__(kThreads) void range_gemm_kernel(const float* __restrict__ E,
                                                              const float* __restrict__ U, int m, int n, int b,
                                                              int c0, int sps, int mtiles, float* __restrict__ P) {
  __shared__ GemmLds lds;
  const int gid = (int)blockIdx.x;
  update_gemm_body(E, U, m, n, b, c0, sps, P, gid % mtiles, gid / mtiles, lds);
}

template <int DT>
__global__ __launch_bounds__(256) void range_reduce_kernel(const void* __restrict__ W, int64_t ldw,
                                                           const int32_t* __restrict__ perm, int m, int n, int b,
                                                           const float* __restrict__ P, int nsplit, int first,
                                                           float* __restrict__ grange) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= m) return;
  const int c0 = b * kBS;
  const int bw = min(kBS, n - c0);
  float mn = INFINITY, mx = -INFINITY;
  for (int c = lane; c < bw; c += 64) {
    const int col = c0 + c;
    const int src = perm != nullptr ? min(max(perm[col], 0), n - 1) : col;
    float v = load_as_f32<DT>(W, r * ldw + src);
    for (int sp = 0; sp < nsplit; ++sp) v -= P[((int64_t)sp * m + r) * kBS + c];
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  if (lane == 0) {
    if (!first) {
      mn = fminf(mn, grange[2 * r]);
      mx = fmaxf(mx, grange[2 * r + 1]);
    }
    grange[2 * r] = mn;
    grange[2 * r + 1] = mx;
  }
}

// The in-block sweep of block kb for 64 rows (4 waves x 16 rows; within a
// wave, lane r < 16 owns row r for the sequential part and all 64 lanes run
// the MFMA part).
// U's diagonal block, upper triangle with the diagonal, packed by rows: row i
// holds columns i .. 127 from offset i (257 - i) / 2 (every read of the sweep
// is on or above the diagonal; half the LDS of a square tile).
constexpr int kUdPacked = kBS * (kBS + 1) / 2;
__device__ __forceinline__ int ud_index(int i, int j) { return i * (2 * kBS + 1 - i) / 2 + (j - i); }

struct SweepLds {
  float Ud[kUdPacked];
  float invd[kBS];
  __attribute__((aligned(16))) float T[kWaves][kRowsPerWave][kTP];
  float Eb[kWaves][kRowsPerWave][kSB + 1];
  float Gs[kWaves][kRowsPerWave][2];
};

// Block kb for rows wg*64 .. wg*64+63.  The block's deferred update arrives
// as nsplit partial products P[sp] (m x 128 each) and, when use_last, the
// product Plast = E[:, block kb-1] U[block kb-1, block kb] that the previous
// block's sweep left for these rows.  When make_next, the rows' errors of
// this block are kept in the tile as its columns are finished and
// E[:, block kb] U[block kb, block kb+1] is written to Plast at the end.
template <int DT, bool SMALLG>
__device__ __forceinline__ void sweep_body(
    const void* __restrict__ Wsrc, int64_t ldw, int m, int n, int kb, const float* __restrict__ U,
    const float* __restrict__ P, int nsplit, float* __restrict__ Plast, int use_last, int make_next, float maxq,
    int g, int G, uint8_t* __restrict__ codes, float* __restrict__ E, float* __restrict__ scales,
    uint8_t* __restrict__ zeros, float* __restrict__ row_loss, int codes_aligned, const int32_t* __restrict__ perm,
    const float* __restrict__ grange, int wg, SweepLds& S) {
  auto& Ud = S.Ud;
  auto& invd = S.invd;
  auto& T = S.T;
  auto& Eb = S.Eb;
  auto& Gs = S.Gs;

  const int c0 = kb * kBS;
  const int bw = min(kBS, n - c0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t row0 = (int64_t)wg * kRowsPerWG + wave * kRowsPerWave;

  // Loads: U's diagonal block (upper triangle, zero below it and beyond bw;
  // 16 float4 slots per thread), the wave's 16 x 128 slab of W and the first
  // kPIn split-K partial products of the block update (P[0] .. P[nsplit-1],
  // then Plast) are all issued before any of them is waited for, so they
  // share one memory round trip; further partials follow kPIn at a time.
  // Slot q of lane l of the slab is row (l + 64q) / 32, columns
  // 4*((l + 64q) % 32) .. +3.
  constexpr int kSlots = kRowsPerWave * kBS / 4 / 64;
  constexpr int kPIn = 2;
  floatx4 t[kSlots];
  {
    const bool vecu = (n & 3) == 0 && (reinterpret_cast<uintptr_t>(U) & 15) == 0;
    constexpr int kUSlots = kBS * kBS / 4 / kThreads;
    // A whole block with aligned rows takes one 16-byte load per U slot and
    // one 16-byte (or, for 16-bit W, 8-byte) load per W slot, with no
    // per-element tests; the lower triangle of the diagonal block is loaded
    // and masked when it is stored to LDS.
    const bool fast = bw == kBS && vecu && perm == nullptr && (ldw & 3) == 0 &&
                      (reinterpret_cast<uintptr_t>(Wsrc) & (DT == GPTQ_F32 ? 15 : 7)) == 0;
    if (fast) {
#pragma unroll
      for (int q = 0; q < kSlots; ++q) {
        const int e = lane + 64 * q;
        const int rr = e >> 5, c = (e & 31) * 4;
        const int64_t row = row0 + rr;
        t[q] = row < m ? load4_as_f32<DT>(Wsrc, row * ldw + c0 + c) : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    } else {
#pragma unroll
      for (int q = 0; q < kSlots; ++q) {
        const int e = lane + 64 * q;
        const int rr = e >> 5, c = (e & 31) * 4;
        const int64_t row = row0 + rr;
        floatx4 v = {0.f, 0.f, 0.f, 0.f};
        if (row < m) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (c + k < bw) {
              // processing position c0 + c + k is original column perm[c0 + c + k]
              const int col = perm != nullptr ? min(max(perm[c0 + c + k], 0), n - 1) : c0 + c + k;
              v[k] = load_as_f32<DT>(Wsrc, row * ldw + col);
            }
        }
        t[q] = v;
      }
    }
    const int nsub = nsplit + (use_last ? 1 : 0);
    auto load_split = [&](int sp, floatx4 (&pv)[kSlots]) {
      const float* src = sp < nsplit ? P + (int64_t)sp * m * kBS : Plast;
#pragma unroll
      for (int q = 0; q < kSlots; ++q) {
        const int e = lane + 64 * q;
        const int rr = e >> 5, c = (e & 31) * 4;
        const int64_t row = row0 + rr;
        pv[q] = (sp < nsub && row < m) ? *reinterpret_cast<const floatx4*>(src + row * kBS + c)
                                       : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    };
    floatx4 pv[kPIn][kSlots];
#pragma unroll
    for (int u = 0; u < kPIn; ++u) load_split(u, pv[u]);
    const float dj = tid < bw ? U[(int64_t)(c0 + tid) * n + c0 + tid] : 1.f;   // kThreads >= kBS
    // U's diagonal block into LDS in two halves of 8 slots (register budget of
    // two workgroups per CU); slots wholly below the diagonal are skipped.
    const bool fullu = bw == kBS && vecu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      floatx4 uv[kUSlots / 2];
#pragma unroll
      for (int q2 = 0; q2 < kUSlots / 2; ++q2) {
        const int e = tid + kThreads * (q2 + h * (kUSlots / 2));
        const int i = e >> 5, j = (e & 31) * 4;
        floatx4 v = {0.f, 0.f, 0.f, 0.f};
        if (j + 3 >= i) {
          const float* p = U + (int64_t)(c0 + i) * n + c0 + j;
          if (fullu) {
            v = *reinterpret_cast<const floatx4*>(p);
          } else if (i < bw) {
            if (vecu && j + 4 <= bw) {
              v = *reinterpret_cast<const floatx4*>(p);
            } else {
#pragma unroll
              for (int k = 0; k < 4; ++k) v[k] = j + k < bw ? p[k] : 0.f;
            }
          }
        }
        uv[q2] = v;
      }
#pragma unroll
      for (int q2 = 0; q2 < kUSlots / 2; ++q2) {
        const int e = tid + kThreads * (q2 + h * (kUSlots / 2));
        const int i = e >> 5, j = (e & 31) * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (j + k >= i) Ud[ud_index(i, j + k)] = uv[q2][k];
      }
    }
    if (tid < kBS) invd[tid] = tid < bw ? 1.f / dj : 0.f;
    for (int sp = 0; sp < nsub; sp += kPIn) {
      if (sp > 0) {
#pragma unroll
        for (int u = 0; u < kPIn; ++u) load_split(sp + u, pv[u]);
      }
#pragma unroll
      for (int u = 0; u < kPIn; ++u)
#pragma unroll
        for (int q = 0; q < kSlots; ++q) t[q] -= pv[u][q];
    }
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const int e = lane + 64 * q;
      const int rr = e >> 5, c = (e & 31) * 4;
      *reinterpret_cast<floatx4*>(&T[wave][rr][c]) = t[q];
    }
  }
  // A group that starts at this block and spans it (g a multiple of 128, or
  // reaching past n): its range is the slab's, reduced across the 32 lanes
  // that hold a row; lanes 0 and 32 of slot q publish rows 2q and 2q + 1.
  const bool block_group = g >= kSB && (c0 % g) == 0 && (g % kBS == 0 || c0 + g >= n);
  // Groups narrower than a register sub-block (1, 2, 4 or 8 columns: SMALLG,
  // a kernel instantiation of its own, so that the other group sizes run
  // code without these starts) begin inside the column chain, which takes
  // their range there from the current values of their columns.
  if (block_group) {
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const int e = lane + 64 * q;
      const int c = (e & 31) * 4;
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k < bw) {
          mn = fminf(mn, t[q][k]);
          mx = fmaxf(mx, t[q][k]);
        }
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 32));
        mx = fmaxf(mx, __shfl_xor(mx, off, 32));
      }
      if ((lane & 31) == 0) {
        Gs[wave][2 * q + (lane >> 5)][0] = mn;
        Gs[wave][2 * q + (lane >> 5)][1] = mx;
      }
    }
  }
  __syncthreads();

  const int r = lane & (kRowsPerWave - 1);
  const int64_t row = row0 + r;
  const bool owner = lane < kRowsPerWave;
  const bool active = owner && row < m;
  float s = 1.f, z = 0.f, inv_s = 1.f;
  // A per-row grid, or a group that began in an earlier block: its grid was
  // stored when the group started.
  if ((g == 0 || (g > kBS && (c0 % g) != 0)) && active) {
    const int gi = g == 0 ? 0 : c0 / g;
    s = scales[row * G + gi];
    z = (float)zeros[row * G + gi];
    inv_s = 1.f / s;
  }
  float loss = 0.f;
  const int nsb = (bw + kSB - 1) / kSB;
  const bool vec_codes = (n & 15) == 0 && codes_aligned;
  const bool vec_e = (n & 3) == 0;

  // One 16-column sub-block: group statistics at a group start, the
  // sequential columns (lane r < 16 owns row r), the codes/E stores and the
  // MFMA push of the sub-block's errors into the block's later columns.  With
  // FULL (a whole 128-column block) sb is a compile-time constant, every loop
  // bound is fixed and the next column's U row is read ahead of the current
  // column's arithmetic.
  // With make_next (whole blocks only), Plast = E[rows, block] U[block,
  // block kb+1] is built as the sweep goes: each wave reads the MFMA B
  // fragments of the off-diagonal tile's 16 rows for sub-block sb straight
  // from global memory at the start of the sub-block (no LDS staging, so the
  // waves never wait for one another), and while it runs sub-block sb+1's
  // columns accumulates sub-block sb's slice E[:, 16] x U_off[16, 128] with
  // 32 fp32 MFMA 16x16x4 (the last slice after the block).
  // The accumulator's columns are permuted so that each lane's B values are
  // four adjacent floats: output tile ct, MFMA column c stands for block
  // column 64*(ct/4) + 4*c + ct%4.  A lane then reads its 32 values of a
  // slice with eight 16-byte loads, and writes Plast with 16-byte stores.
  const int c0n = c0 + kBS;
  const int bwn = min(kBS, n - c0n);
  floatx4 pacc[kBS / 16];
#pragma unroll
  for (int ct = 0; ct < kBS / 16; ++ct) pacc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  const bool vec_uo = (n & 3) == 0 && (reinterpret_cast<uintptr_t>(U) & 15) == 0;
  // uf[k4][h][t]: B element (k = 4*k4 + lane/16) of tile ct = 4*h + t, i.e.
  // U_off[k, 64*h + 4*(lane%16) + t].
  floatx4 uf[kSB / 4][2];
  auto uoff_load = [&](int j0, floatx4 (&f)[kSB / 4][2]) {
#pragma unroll
    for (int k4 = 0; k4 < kSB / 4; ++k4) {
      const float* p = U + (int64_t)(c0 + j0 + 4 * k4 + (lane >> 4)) * n + c0n + 4 * (lane & 15);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 64 * h + 4 * (lane & 15);
        floatx4 v = {0.f, 0.f, 0.f, 0.f};
        if (vec_uo && c + 4 <= bwn) {
          v = *reinterpret_cast<const floatx4*>(p + 64 * h);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = c + t < bwn ? p[64 * h + t] : 0.f;
        }
        f[k4][h] = v;
      }
    }
  };
  auto uoff_accumulate = [&](int j0, const floatx4 (&f)[kSB / 4][2]) {
#pragma unroll
    for (int k4 = 0; k4 < kSB / 4; ++k4) {
      const float a = T[wave][lane & 15][j0 + 4 * k4 + (lane >> 4)];
#pragma unroll
      for (int ct = 0; ct < kBS / 16; ++ct)
        pacc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, f[k4][ct >> 2][ct & 3], pacc[ct], 0, 0, 0);
    }
  };

  // A group of g < 16 columns starts at processing column col (sub-block
  // column jj): its range is over the current values w[jj .. jj+g) of this
  // row (columns from `lim` on lie past the layer), then its grid is stored.
  // Called with a compile-time jj from the unrolled chains, so w stays in
  // registers.
  auto small_group_start = [&](int col, int jj, const float (&wv)[kSB], int lim) {
    float mn = wv[jj], mx = wv[jj];
#pragma unroll
    for (int kk = 1; kk < kSB; ++kk) {
      if (jj + kk < kSB && kk < g && jj + kk < lim) {
        mn = fminf(mn, wv[jj + kk]);
        mx = fmaxf(mx, wv[jj + kk]);
      }
    }
    grid_from_range(mn, mx, maxq, s, z, inv_s);
    if (active) {
      const int gi = col / g;
      scales[row * G + gi] = s;
      zeros[row * G + gi] = (uint8_t)z;
    }
  };

  auto sub_block = [&](auto sbc, auto fullc) {
    constexpr bool FULL = decltype(fullc)::value;
    const int sb = sbc;
    const int j0 = sb * kSB;
    if constexpr (FULL) {
      // the fragments of the previous sub-block's slice (all zero, and no
      // access, when there is no next block); consumed from column 8 on
      if (sb > 0) uoff_load(j0 - kSB, uf);
    }
    if (block_group && sb == 0) {
      float gmn = Gs[wave][r][0], gmx = Gs[wave][r][1];
      if (g > kBS && c0 + kBS < n && active) {
        // the group goes on past this block: fold in its later blocks' range
        gmn = fminf(gmn, grange[2 * row]);
        gmx = fmaxf(gmx, grange[2 * row + 1]);
      }
      grid_from_range(gmn, gmx, maxq, s, z, inv_s);
      if (active) {
        const int gi = c0 / g;
        scales[row * G + gi] = s;
        zeros[row * G + gi] = (uint8_t)z;
      }
    } else if (g >= kSB && ((c0 + j0) % g) == 0) {
      // group range over the current values; g is a multiple of 16 and the
      // group lies inside the block (tail columns beyond bw are excluded)
      const int gl = min(g, bw - j0);
      float mn = T[wave][r][j0], mx = mn;
      for (int c4 = 0; c4 < g; c4 += 16) {
        floatx4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const floatx4*>(&T[wave][r][j0 + c4 + 4 * u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (c4 + 4 * u + k < gl) {
              mn = fminf(mn, v[u][k]);
              mx = fmaxf(mx, v[u][k]);
            }
      }
      grid_from_range(mn, mx, maxq, s, z, inv_s);
      if (active) {
        const int gi = (c0 + j0) / g;
        scales[row * G + gi] = s;
        zeros[row * G + gi] = (uint8_t)z;
      }
    }
    float w[kSB];
#pragma unroll
    for (int jj = 0; jj < kSB; ++jj) w[jj] = T[wave][r][j0 + jj];
    float eb[kSB];
    uint32_t cw[kSB / 4] = {0u, 0u, 0u, 0u};
    if constexpr (FULL) {
      float un[kSB];
      float idn = invd[j0];
#pragma unroll
      for (int kk = 0; kk < kSB; ++kk) un[kk] = Ud[ud_index(j0, j0 + kk)];
      // The previous sub-block's Plast slice (independent of this chain) is
      // spread over the second half of the columns, four MFMAs per column,
      // so that the matrix core works while the column chain waits on its
      // own latencies and the fragments' loads have eight columns to land.
      constexpr bool kSlice = decltype(sbc)::value > 0;
      float pa[kSB / 4];
      if constexpr (kSlice) {
#pragma unroll
        for (int k4 = 0; k4 < kSB / 4; ++k4) pa[k4] = T[wave][lane & 15][j0 - kSB + 4 * k4 + (lane >> 4)];
      }
#pragma unroll
      for (int jj = 0; jj < kSB; ++jj) {
        if constexpr (kSlice) {
          if (jj >= kSB / 2) {
            const int k4 = (jj - kSB / 2) >> 1, h = (jj - kSB / 2) & 1;
#pragma unroll
            for (int t = 0; t < 4; ++t)
              pacc[4 * h + t] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k4], uf[k4][h][t], pacc[4 * h + t], 0, 0, 0);
          }
        }
        float uc[kSB];
#pragma unroll
        for (int kk = 0; kk < kSB; ++kk) uc[kk] = un[kk];
        const float idc = idn;
        if (jj + 1 < kSB) {
          idn = invd[j0 + jj + 1];
#pragma unroll
          for (int kk = jj + 2; kk < kSB; ++kk) un[kk] = Ud[ud_index(j0 + jj + 1, j0 + kk)];
        }
        if constexpr (SMALLG) {
          if (((c0 + j0 + jj) & (g - 1)) == 0) small_group_start(c0 + j0 + jj, jj, w, kSB);
        }
        const float c = quant_code(w[jj], s, inv_s, z, maxq);
        const float what = s * (c - z);
        const float e = (w[jj] - what) * idc;
        eb[jj] = active ? e : 0.f;
        loss = __builtin_fmaf(e, e, loss);
        cw[jj >> 2] |= (uint32_t)c << (8 * (jj & 3));
#pragma unroll
        for (int kk = jj + 1; kk < kSB; ++kk) w[kk] = __builtin_fmaf(-e, uc[kk], w[kk]);
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < kSB; ++jj) {
        if (j0 + jj < bw) {
          if constexpr (SMALLG) {
            if (((c0 + j0 + jj) & (g - 1)) == 0) small_group_start(c0 + j0 + jj, jj, w, bw - j0);
          }
          const float c = quant_code(w[jj], s, inv_s, z, maxq);
          const float what = s * (c - z);
          const float e = (w[jj] - what) * invd[j0 + jj];
          eb[jj] = active ? e : 0.f;
          loss = __builtin_fmaf(e, e, loss);
          cw[jj >> 2] |= (uint32_t)c << (8 * (jj & 3));
#pragma unroll
          for (int kk = jj + 1; kk < kSB; ++kk) w[kk] = __builtin_fmaf(-e, Ud[ud_index(j0 + jj, j0 + kk)], w[kk]);
        } else {
          eb[jj] = 0.f;
        }
      }
    }
    if (active) {
      uint8_t* cp = codes + row * n + c0 + j0;
      float* ep = E + row * n + c0 + j0;
      if (j0 + kSB <= bw && vec_codes) {
        *reinterpret_cast<u32x4*>(cp) = u32x4{cw[0], cw[1], cw[2], cw[3]};
      } else {
        for (int jj = 0; jj < kSB && j0 + jj < bw; ++jj) cp[jj] = (uint8_t)(cw[jj >> 2] >> (8 * (jj & 3)));
      }
      if (j0 + kSB <= bw && vec_e) {
#pragma unroll
        for (int q = 0; q < kSB / 4; ++q)
          reinterpret_cast<floatx4*>(ep)[q] = floatx4{eb[4 * q], eb[4 * q + 1], eb[4 * q + 2], eb[4 * q + 3]};
      } else {
        for (int jj = 0; jj < kSB && j0 + jj < bw; ++jj) ep[jj] = eb[jj];
      }
    }
    if (owner) {
#pragma unroll
      for (int jj = 0; jj < kSB; ++jj) Eb[wave][r][jj] = eb[jj];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Push the sub-block's errors into the block's later columns:
    // T[:, ct] -= Eb * Ud[j0:j0+16, ct] for each later 16-column tile ct.
    // 16x16x4 accumulator: register i of lane l is row 4*(l/16) + i, column l%16.
    auto push_tile = [&](int ct) {
      floatx4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = T[wave][4 * (lane >> 4) + i][ct * kSB + (lane & 15)];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int k = k4 * 4 + (lane >> 4);
        const float a = -Eb[wave][lane & 15][k];
        const float b = Ud[ud_index(j0 + k, ct * kSB + (lane & 15))];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) T[wave][4 * (lane >> 4) + i][ct * kSB + (lane & 15)] = acc[i];
    };
    if constexpr (FULL) {
#pragma unroll
      for (int ct = sbc + 1; ct < kBS / kSB; ++ct) push_tile(ct);
    } else {
      for (int ct = sb + 1; ct < nsb; ++ct) push_tile(ct);
    }
    // The sub-block's columns are finished: keep their errors in the tile.
    if (make_next && owner) {
#pragma unroll
      for (int q = 0; q < kSB / 4; ++q)
        *reinterpret_cast<floatx4*>(&T[wave][r][j0 + 4 * q]) = floatx4{eb[4 * q], eb[4 * q + 1], eb[4 * q + 2], eb[4 * q + 3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (bw == kBS) {
    static_for<kBS / kSB>([&](auto sbc) { sub_block(sbc, std::true_type{}); });
  } else {
    for (int sb = 0; sb < nsb; ++sb) sub_block(sb, std::false_type{});
  }
  if (active && row_loss != nullptr) row_loss[row] = (kb == 0 ? 0.f : row_loss[row]) + 0.5f * loss;
  if (make_next) {
    // Last slice, then Plast[rows] = E[rows, block kb] U[block kb, block kb+1].
    uoff_load(kBS - kSB, uf);
    uoff_accumulate(kBS - kSB, uf);
    // 16x16x4 accumulator: register i of lane l is row 4*(l/16) + i, MFMA
    // column l%16, so tiles 4h .. 4h+3 hold block columns 64h + 4*(l%16) + 0..3.
    const bool vec_pl = (reinterpret_cast<uintptr_t>(Plast) & 15) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t grow = row0 + 4 * (lane >> 4) + i;
      if (grow >= m) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float* d = Plast + grow * kBS + 64 * h + 4 * (lane & 15);
        const floatx4 v = {pacc[4 * h][i], pacc[4 * h + 1][i], pacc[4 * h + 2][i], pacc[4 * h + 3][i]};
        if (vec_pl) {
          *reinterpret_cast<floatx4*>(d) = v;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) d[t] = v[t];
        }
      }
    }
  }
}

// One launch per block kb: workgroups 0 .. nsw-1 sweep block kb (64 rows
// each); workgroups nsw .. compute the partial products of block kb+1's
// deferred update over the columns before block kb (the last block's share
// comes from the sweep itself), split over K in ranges of sps stages.
template <int DT, bool SMALLG>
__global__ __launch_bounds__(kThreads, 2) void quant_block_kernel(
    const void* __restrict__ Wsrc, int64_t ldw, int m, int n, int kb, const float* __restrict__ U,
    const float* __restrict__ Pcur, int nsplit, float* __restrict__ Plast, int use_last, int make_next,
    float maxq, int g, int G, uint8_t* __restrict__ codes, float* __restrict__ E, float* __restrict__ scales,
    uint8_t* __restrict__ zeros, float* __restrict__ row_loss, int codes_aligned, const int32_t* __restrict__ perm,
    const float* __restrict__ grange, int nsw, int mtiles, int sps, float* __restrict__ Pnext) {
  __shared__ union {
    SweepLds s;
    GemmLds g;
  } lds;
  const int wg = (int)blockIdx.x;
  if (wg < nsw) {
    sweep_body<DT, SMALLG>(Wsrc, ldw, m, n, kb, U, Pcur, nsplit, Plast, use_last, make_next, maxq, g, G, codes, E,
                           scales, zeros, row_loss, codes_aligned, perm, grange, wg, lds.s);
  } else {
    const int gid = wg - nsw;
    update_gemm_body(E, U, m, n, kb + 1, kb * kBS, sps, Pnext, gid % mtiles, gid / mtiles, lds.g);
  }
}

struct QuantLayout {
  int nblocks = 0, mtiles = 0, nsw = 0, smax = 0;
  size_t off_E = 0, off_P = 0, off_Plast = 0, off_pinv = 0, off_grange = 0, pstride = 0, total = 0;
};

// Number of K splits of block kb+1's update (over `stages` 32-column stages)
// that finishes the launch soonest.  One workgroup of either role occupies a
// CU (the LDS of the sweep role); the nsw sweep workgroups are dispatched
// first and take about kSweepUs each; an update workgroup takes kStageUs per
// stage plus kItemUs.  Greedy list scheduling of identical items on 256 CUs
// gives the launch time in closed form; the fewest splits within 1% of the
// best are taken (fewer partial products for the sweep to read).
constexpr double kSweepUs = 35.0, kStageUs = 2.5, kItemUs = 3.0;
constexpr int kMaxSplits = 16;

int choose_splits(int nsw, int mtiles, int stages) {
  if (stages <= 0) return 0;
  const int cus = 256;
  const int q = nsw / cus, a = nsw % cus;           // sweeps per CU: q, or q + 1 on a CUs
  double best = 1e300;
  double cost[kMaxSplits + 1];
  const int smax = std::min(stages, kMaxSplits);
  for (int S = 1; S <= smax; ++S) {
    const int sps = (int)ceil_div(stages, S);
    const int items = (int)ceil_div(stages, sps) * mtiles;
    const double d = sps * kStageUs + kItemUs;
    const int full = items / cus, rem = items % cus;
    // CUs free at q * kSweepUs (256 - a of them) take the remainder first.
    const int early = cus - a;
    double t = q * kSweepUs + (full + (rem > 0 ? 1 : 0)) * d;
    if (a > 0) t = std::max(t, (q + 1) * kSweepUs + (full + (rem > early ? 1 : 0)) * d);
    cost[S] = t;
    best = std::min(best, t);
  }
  for (int S = 1; S <= smax; ++S)
    if (cost[S] <= best * 1.01) return S;
  return 1;
}

// Workspace: E (m x n float32 scaled errors), two buffers of split-K partial
// products (smax x m x 128 float32 each), Plast (m x 128), the inverse
// permutation (n int32) and the per-row ranges of wide groups (m x 2 float32).
QuantLayout quant_layout(int64_t m, int64_t n) {
  QuantLayout L;
  L.nblocks = (int)ceil_div(n, kBS);
  L.mtiles = (int)ceil_div(m, 128);
  L.nsw = (int)ceil_div(m, kRowsPerWG);
  // The most partial products any launch writes (at least one buffer row);
  // the group-range products of wide groups use a single split per K range
  // of the same size, so they fit as well.
  L.smax = 1;
  for (int kb = 1; kb + 1 < L.nblocks; ++kb) {
    const int stages = kb * (kBS / kUK);
    const int S = choose_splits(L.nsw, L.mtiles, stages);
    const int sps = (int)ceil_div(stages, S);
    L.smax = std::max(L.smax, (int)ceil_div(stages, sps));
  }
  const size_t mn = (size_t)m * (size_t)n * sizeof(float);
  L.pstride = (size_t)L.smax * (size_t)m * kBS;   // floats per partial-product buffer
  L.off_E = 0;
  L.off_P = align256(L.off_E + mn);
  L.off_Plast = align256(L.off_P + 2 * L.pstride * sizeof(float));
  L.off_pinv = align256(L.off_Plast + (size_t)m * kBS * sizeof(float));
  L.off_grange = align256(L.off_pinv + (size_t)n * sizeof(int32_t));
  L.total = align256(L.off_grange + (size_t)m * 2 * sizeof(float));
  return L;
}

template <int DT>
gptq_status launch_block(const void* src, int64_t ld, int m, int n, int kb, const float* U, const float* Pcur,
                         int nsplit, float* Plast, int use_last, int make_next, float maxq, int g, int G,
                         uint8_t* codes, float* E, float* scales, uint8_t* zeros, float* row_loss,
                         const int32_t* perm, const float* grange, int nsw, int mtiles, int ngemm, int sps,
                         float* Pnext, hipStream_t st) {
  const int codes_aligned = (reinterpret_cast<uintptr_t>(codes) & 15) == 0;
  auto kern = g > 0 && g < kSB ? quant_block_kernel<DT, true> : quant_block_kernel<DT, false>;
  kern<<<(unsigned)(nsw + ngemm), kThreads, 0, st>>>(src, ld, m, n, kb, U, Pcur, nsplit, Plast, use_last, make_next,
                                                      maxq, g, G, codes, E, scales, zeros, row_loss, codes_aligned,
                                                      perm, grange, nsw, mtiles, sps, Pnext);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

// The range of the later blocks of a group that starts at block kb and spans
// gb blocks, over their values at the group start (into grange).
template <int DT>
gptq_status launch_group_range(const void* W, int64_t ldw, const int32_t* perm, int m, int n, int kb, int gb,
                               const float* E, const float* U, float* Ptmp, int mtiles, int smax, float* grange,
                               hipStream_t st) {
  const int c0 = kb * kBS;
  const int nblocks = (int)ceil_div(n, kBS);
  bool first = true;
  for (int b = kb + 1; b < std::min(nblocks, kb + gb); ++b) {
    const int stages = c0 / kUK;
    int nsplit = 0;
    if (stages > 0) {
      // at most smax splits: Ptmp holds smax partial products
      const int S = std::min(smax, std::max(1, choose_splits(0, mtiles, stages)));
      const int sps = (int)ceil_div(stages, S);
      nsplit = (int)ceil_div(stages, sps);
      range_gemm_kernel<<<(unsigned)(mtiles * nsplit), kThreads, 0, st>>>(E, U, m, n, b, c0, sps, mtiles, Ptmp);
      GPTQ_TRY_LAUNCH();
    }
    range_reduce_kernel<DT><<<(unsigned)ceil_div(m, 4), 256, 0, st>>>(W, ldw, perm, m, n, b, Ptmp, nsplit,
                                                                      first ? 1 : 0, grange);
    GPTQ_TRY_LAUNCH();
    first = false;
  }
  return GPTQ_OK;
}

template <int DT>
gptq_status launch_row_grid(const void* W, int64_t ldw, int m, int n, float maxq, float* scales, uint8_t* zeros,
                            hipStream_t st) {
  row_grid_kernel<DT><<<(unsigned)ceil_div(m, 4), 256, 0, st>>>(W, ldw, m, n, maxq, scales, zeros);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

template <int DT>
gptq_status quantize_typed(const void* W, int64_t ldw, int m, int n, const float* U, const int32_t* perm,
                           int levels, int g, uint8_t* codes, float* scales, uint8_t* zeros, int32_t* g_idx,
                           float* row_loss, void* Wq, const QuantLayout& L, char* base, hipStream_t st) {
  float* E = reinterpret_cast<float*>(base + L.off_E);
  float* P = reinterpret_cast<float*>(base + L.off_P);
  float* Plast = reinterpret_cast<float*>(base + L.off_Plast);
  int32_t* pinv = reinterpret_cast<int32_t*>(base + L.off_pinv);
  float* grange = reinterpret_cast<float*>(base + L.off_grange);
  const float maxq = (float)(levels - 1);
  const int G = g == 0 ? 1 : (int)ceil_div(n, g);

  if (perm != nullptr || g_idx != nullptr) {
    index_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, st>>>(n, perm, g, perm != nullptr ? pinv : nullptr, g_idx);
    GPTQ_TRY_LAUNCH();
  }
  if (g == 0) {
    const gptq_status rc = launch_row_grid<DT>(W, ldw, m, n, maxq, scales, zeros, st);
    if (rc != GPTQ_OK) return rc;
  }
  int ns_cur = 0;   // partial products of block kb's update, from the previous launch
  for (int kb = 0; kb < L.nblocks; ++kb) {
    const int use_last = kb >= 1;
    const int make_next = kb + 1 < L.nblocks;
    const float* Pcur = P + (size_t)(kb & 1) * L.pstride;
    float* Pnext = P + (size_t)((kb + 1) & 1) * L.pstride;
    if (g > kBS && (kb * kBS) % g == 0 && make_next) {
      // Pnext is free until this block's launch writes it.
      const gptq_status rc = launch_group_range<DT>(W, ldw, perm, m, n, kb, g / kBS, E, U, Pnext, L.mtiles,
                                                    L.smax, grange, st);
      if (rc != GPTQ_OK) return rc;
    }
    int ns_next = 0, sps = 0;
    if (make_next && kb >= 1) {
      // Block kb+1's update over columns [0, 128 kb) in ranges of whole 32-column stages.
      const int stages = kb * (kBS / kUK);
      const int s_target = choose_splits(L.nsw, L.mtiles, stages);
      sps = (int)ceil_div(stages, s_target);
      ns_next = (int)ceil_div(stages, sps);
    }
    const int ngemm = L.mtiles * ns_next;
    const gptq_status rc = launch_block<DT>(W, ldw, m, n, kb, U, Pcur, ns_cur, Plast, use_last, make_next, maxq, g,
                                            G, codes, E, scales, zeros, row_loss, perm, grange, L.nsw, L.mtiles,
                                            ngemm, sps, Pnext, st);
    if (rc != GPTQ_OK) return rc;
    ns_cur = ns_next;
  }
  if (perm != nullptr || Wq != nullptr) {
    const size_t shm = perm != nullptr ? (size_t)n : 0;
    finalize_kernel<DT><<<(unsigned)m, 256, shm, st>>>(codes, n, perm != nullptr ? pinv : nullptr, scales, zeros, g,
                                                       G, Wq, n);
    GPTQ_TRY_LAUNCH();
  }
  return GPTQ_OK;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_quantize_ws_bytes(int64_t m, int64_t n, int block_size) {
  if (m <= 0 || n <= 0 || block_size != kBS) return 0;
  return quant_layout(m, n).total;
}

extern "C" gptq_status gptq_quantize_layer(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw,
                                           const float* U, const int32_t* perm, int levels, int group_size,
                                           int block_size, uint8_t* codes, float* scales, uint8_t* zeros,
                                           int32_t* g_idx, float* row_loss, void* Wq, void* ws, size_t ws_bytes,
                                           void* stream) {
  if (m < 0 || n < 0 || !valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (!(levels == 3 || levels == 4 || levels == 8 || levels == 16)) return GPTQ_ERR_INVALID_ARG;
  if (group_size < 0 || block_size <= 0) return GPTQ_ERR_INVALID_ARG;
  if (block_size != kBS) return GPTQ_ERR_UNSUPPORTED;
  // groups that divide the block (the 16-column register sub-block included)
  // or are whole multiples of it
  if (!(group_size == 0 || kBS % group_size == 0 || group_size % kBS == 0)) return GPTQ_ERR_UNSUPPORTED;
  if (n > (int64_t)1 << 16 || m > ((int64_t)1 << 31) - 1) return GPTQ_ERR_UNSUPPORTED;
  if (n == 0) return GPTQ_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (m == 0) {
    if (g_idx == nullptr) return GPTQ_OK;
    index_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, st>>>((int)n, perm, group_size, nullptr, g_idx);
    GPTQ_TRY_LAUNCH();
    return GPTQ_OK;
  }
  if (W == nullptr || U == nullptr || codes == nullptr || scales == nullptr || zeros == nullptr || ldw < n)
    return GPTQ_ERR_INVALID_ARG;
  const QuantLayout L = quant_layout(m, n);
  if (ws == nullptr || ws_bytes < L.total) return GPTQ_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  const int mi = (int)m, ni = (int)n;
  if (w_dtype == GPTQ_F32)
    return quantize_typed<GPTQ_F32>(W, ldw, mi, ni, U, perm, levels, group_size, codes, scales, zeros, g_idx,
                                    row_loss, Wq, L, base, st);
  if (w_dtype == GPTQ_F16)
    return quantize_typed<GPTQ_F16>(W, ldw, mi, ni, U, perm, levels, group_size, codes, scales, zeros, g_idx,
                                    row_loss, Wq, L, base, st);
  return quantize_typed<GPTQ_BF16>(W, ldw, mi, ni, U, perm, levels, group_size, codes, scales, zeros, g_idx,
                                   row_loss, Wq, L, base, st);
}
