// Reading the packed weights back: Y = X W^T straight from the packed codes,
// for decode-sized batches.
// GPTQ knowledge note, "Tradeoffs": the speed of a quantized model rests on
// kernels that consume the packed weights, inference being limited by weight
// memory traffic; anthology record SOTA-185, "The scope worth holding onto":
// decode is bandwidth-bound.
//
//   Y[b, r] = sum_k s[r, g_k] (c[r, k] - z[r, g_k]) X[b, k]
//
// One wave owns kRows rows; lane l walks the row's 32-column segments l,
// l + 64, ...  A segment is `bits` consecutive words of a row.  Its codes are
// turned into float16 subnormals c * 2^-24 (a b-bit code is exactly the
// mantissa of a subnormal whose exponent field is 0), two per register, and
// multiplied into float32 by v_dot2_f32_f16 against the same two columns of
// X, so decoding costs about one masked shift per two codes.  Codes are
// paired as (c_i, c_{i+H}) with H = 4 (4-bit), 8 (2-bit) or 16 (3-bit) so
// that one shift and one mask extract a pair; the matching X pairs are
// rearranged once per segment (v_perm_b32) and shared by the wave's rows.
// When the 32 columns of a segment share one group (per-row grids, or
// contiguous groups of a multiple of 32 columns):
//   y += s * (2^24 * sum_k c_k x_k - z * sum_k x_k)
// with sum x formed once per segment.  Otherwise (g_idx given, or groups not a
// multiple of 32) each code takes its own group: y += s_g (c - z_g) x in
// float32.
#include "common.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Rows per wave (8 for small batches was measured: no faster on the large
// layer, slower on small ones).
template <int NB> constexpr int rows_per_wave() { return 4; }
constexpr int kSeg = 32;  // columns per lane segment
constexpr float kTwo24 = 16777216.0f;
constexpr int64_t kGridCap = 2048;            // workgroups at most (8 per CU)
constexpr size_t kMaxStageBytes = 64 * 1024;  // LDS for staged (s, s*z) pairs
constexpr int kXregMaxSpl = 6;                // decode kernel with X in registers: n <= 64 * 32 * 6
constexpr int64_t kXregGrid = 768;             // its workgroups (three per CU), waves stream rows

typedef __fp16 half2_t __attribute__((ext_vector_type(2)));

// X pair (x_a, x_{a+H}) from the natural pairs xn[t] = (x_{2t}, x_{2t+1});
// H is even, so both halves come from the same position of their pair.
__device__ inline uint32_t x_pair(const uint32_t (&xn)[kSeg / 2], int a, int h) {
  const uint32_t lo = xn[a >> 1], hi = xn[(a + h) >> 1];
  return __builtin_amdgcn_perm(hi, lo, (a & 1) ? 0x07060302u : 0x05040100u);
}

// Code pairs of one segment, pair j = (c_{a_j}, c_{a_j + H}) as two float16
// subnormals; a_j and H follow the bit width.
template <int BITS> struct Decode;

template <> struct Decode<4> {
  static constexpr int H = 4;
  __device__ static int first(int j) { return 8 * (j >> 2) + (j & 3); }
  __device__ static uint32_t pair(const uint32_t (&w)[4], int j) { return (w[j >> 2] >> (4 * (j & 3))) & 0x000F000Fu; }
  __device__ static void pairs(const uint32_t (&w)[4], uint32_t (&p)[kSeg / 2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[4 * q + i] = (w[q] >> (4 * i)) & 0x000F000Fu;
  }
};

template <> struct Decode<2> {
  static constexpr int H = 8;
  __device__ static int first(int j) { return 16 * (j >> 3) + (j & 7); }
  __device__ static uint32_t pair(const uint32_t (&w)[2], int j) { return (w[j >> 3] >> (2 * (j & 7))) & 0x00030003u; }
  __device__ static void pairs(const uint32_t (&w)[2], uint32_t (&p)[kSeg / 2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) p[8 * q + i] = (w[q] >> (2 * i)) & 0x00030003u;
  }
};

template <> struct Decode<3> {
  static constexpr int H = 16;
  __device__ static int first(int j) { return j; }
  __device__ static uint32_t pair(const uint32_t (&w)[3], int j) {
    const uint64_t lo = (uint64_t)w[0] | ((uint64_t)(w[1] & 0xFFFFu) << 32);
    const uint64_t hi = (uint64_t)(w[1] >> 16) | ((uint64_t)w[2] << 16);
    return (uint32_t)((lo >> (3 * j)) & 7u) | ((uint32_t)((hi >> (3 * j)) & 7u) << 16);
  }
  __device__ static void pairs(const uint32_t (&w)[3], uint32_t (&p)[kSeg / 2]) {
    // bits 0..47 hold codes 0..15, bits 48..95 codes 16..31
    const uint64_t lo = (uint64_t)w[0] | ((uint64_t)(w[1] & 0xFFFFu) << 32);
    const uint64_t hi = (uint64_t)(w[1] >> 16) | ((uint64_t)w[2] << 16);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      p[i] = (uint32_t)((lo >> (3 * i)) & 7u) | ((uint32_t)((hi >> (3 * i)) & 7u) << 16);
  }
};

// Code k (0..31) of a segment from its words.
template <int BITS>
__device__ inline uint32_t code_at(const uint32_t (&w)[BITS], int k) {
  const int bit = k * BITS, q = bit >> 5, off = bit & 31;
  uint32_t v = w[q] >> off;
  if (off + BITS > 32) v |= w[q + 1] << (32 - off);
  return v & ((1u << BITS) - 1u);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// NB = batch rows of X handled (a multiple of the runtime batch's round-up);
// PER_CODE selects the per-code group path.
template <int BITS, int NB, bool PER_CODE>
__global__ __launch_bounds__(kThreads) void dequant_gemv_kernel(
    const uint32_t* __restrict__ packed, int m, int n, int64_t ldp, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int G, int group_size, const int32_t* __restrict__ g_idx,
    const uint16_t* __restrict__ X, int batch, int64_t ldx, float* __restrict__ Y, int64_t ldy, int vec_w,
    int vec_x, int stage_sz) {
  using D = Decode<BITS>;
  constexpr int kRows = rows_per_wave<NB>();
  extern __shared__ float2 sz_lds[];  // per wave: kRows x G pairs (s, s*z), per-code path
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nseg = (n + kSeg - 1) / kSeg;
  const int nw = (int)(((int64_t)n * BITS + 31) / 32);  // words per row
  const int ngroups = (m + kRows - 1) / kRows;
  for (int rg = (int)blockIdx.x * kWaves + wave; rg < ngroups; rg += (int)gridDim.x * kWaves) {
  const int r0 = rg * kRows;
  float2* szw = sz_lds + (size_t)wave * kRows * G;
  if constexpr (PER_CODE) {
    if (stage_sz) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int e = lane; e < kRows * G; e += 64) {
        const int rr = e / G, gg = e - rr * G;
        const int r = r0 + rr < m ? r0 + rr : m - 1;
        const float sc = scales[(int64_t)r * G + gg];
        szw[e] = make_float2(sc, sc * (float)zeros[(int64_t)r * G + gg]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  float yacc[kRows][NB];
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
    for (int b = 0; b < NB; ++b) yacc[rr][b] = 0.f;

  for (int seg = lane; seg < nseg; seg += 64) {
    const int k0 = seg * kSeg;
    const bool whole = k0 + kSeg <= n;
    // X of the segment: natural f16 pairs per batch row (zero past n and past batch).
    uint32_t xn[NB][kSeg / 2];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint16_t* xr = X + (int64_t)(b < batch ? b : 0) * ldx + k0;
      if (b < batch && whole && vec_x) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(xr + 8 * v);
#pragma unroll
          for (int e = 0; e < 4; ++e) xn[b][4 * v + e] = t[e];
        }
      } else {
#pragma unroll
        for (int t = 0; t < kSeg / 2; ++t) {
          const uint32_t lo = (b < batch && k0 + 2 * t < n) ? xr[2 * t] : 0u;
          const uint32_t hi = (b < batch && k0 + 2 * t + 1 < n) ? xr[2 * t + 1] : 0u;
          xn[b][t] = lo | (hi << 16);
        }
      }
    }
    if constexpr (!PER_CODE) {
      // X pairs in decode order and the segment sums of X.
      uint32_t xq[NB][kSeg / 2];
      float xs[NB];
      const uint32_t ones = 0x3C003C00u;  // (1.0, 1.0) in float16
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        xs[b] = 0.f;
#pragma unroll
        for (int j = 0; j < kSeg / 2; ++j) {
          xq[b][j] = x_pair(xn[b], D::first(j), D::H);
          xs[b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, xn[b][j]),
                                         __builtin_bit_cast(half2_t, ones),
                                         xs[b], false);
        }
      }
      const int g = group_size > 0 ? k0 / group_size : 0;
#pragma unroll
      for (int rr = 0; rr < kRows; ++rr) {
        const int r = r0 + rr;
        if (r >= m) break;
        const uint32_t* wr = packed + (int64_t)r * ldp + (int64_t)seg * BITS;
        uint32_t w[BITS];
        if (whole && vec_w && BITS != 3) {
          if constexpr (BITS == 4) {
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr));
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = t[e];
          } else if constexpr (BITS == 2) {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(wr));
            w[0] = t[0];
            w[1] = t[1];
          }
        } else {
#pragma unroll
          for (int e = 0; e < BITS; ++e) w[e] = seg * BITS + e < nw ? __builtin_nontemporal_load(wr + e) : 0u;
        }
        uint32_t p[kSeg / 2];
        D::pairs(w, p);
        const float s = scales[(int64_t)r * G + g];
        const float z = (float)zeros[(int64_t)r * G + g];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < kSeg / 2; ++j)
            a = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, p[j]),
                                       __builtin_bit_cast(half2_t, xq[b][j]),
                                       a, false);
          yacc[rr][b] = __builtin_fmaf(s, __builtin_fmaf(a, kTwo24, -z * xs[b]), yacc[rr][b]);
        }
      }
    } else {
      // Each code its own group.
      uint32_t w[kRows][BITS];
#pragma unroll
      for (int rr = 0; rr < kRows; ++rr) {
        const uint32_t* wr = packed + (int64_t)(r0 + rr < m ? r0 + rr : r0) * ldp + (int64_t)seg * BITS;
#pragma unroll
        for (int e = 0; e < BITS; ++e) w[rr][e] = seg * BITS + e < nw ? wr[e] : 0u;
      }
#pragma unroll
      for (int k = 0; k < kSeg; ++k) {
        const int col = k0 + k < n ? k0 + k : n - 1;
        const int gk = g_idx != nullptr ? g_idx[col] : (group_size > 0 ? col / group_size : 0);
        float xk[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
          xk[b] = (float)__builtin_bit_cast(_Float16, (uint16_t)(xn[b][k >> 1] >> (16 * (k & 1))));
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) {
          const int r = r0 + rr;
          if (r >= m) break;
          const float c = (float)code_at<BITS>(w[rr], k);
          float2 q;
          if (stage_sz) {
            q = szw[rr * G + gk];
          } else {
            const float sc = scales[(int64_t)r * G + gk];
            q = make_float2(sc, sc * (float)zeros[(int64_t)r * G + gk]);
          }
          // s (c - z) x as c (s x) - (s z) x
#pragma unroll
          for (int b = 0; b < NB; ++b)
            yacc[rr][b] = __builtin_fmaf(c, q.x * xk[b], __builtin_fmaf(-q.y, xk[b], yacc[rr][b]));
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = wave_sum(yacc[rr][b]);
      if (lane == 0 && r0 + rr < m && b < batch) Y[(int64_t)b * ldy + r0 + rr] = v;
    }
  }
}


// Decode (NB = 1 or 2 rows of X), segments that share one group, aligned
// rows: lane l owns the segments l, l + 64, ... of every row — the same
// columns of X for all rows — so the X pairs of each segment (in decode
// order) and their sums are formed once per workgroup into LDS (pair j of a
// segment at [b][slot][j][lane]: a wave's reads are conflict-free) and the
// waves stream rows, loading the next row's words and grid values while the
// current row is multiplied.  Per lane and X row the accumulation over the
// lane's segments and the wave sum are those of dequant_gemv_kernel, so Y is
// the same.  SPL = segments per lane (n <= 64 * 32 * SPL); n a multiple of 32.
template <int BITS, int SPL, int NB>
__global__ __launch_bounds__(kThreads) void dequant_gemv_xreg_kernel(
    const uint32_t* __restrict__ packed, int m, int n, int64_t ldp, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int G, int group_size, const uint16_t* __restrict__ X, int64_t ldx,
    float* __restrict__ Y, int64_t ldy) {
  static_assert(BITS == 2 || BITS == 4, "whole-word segments");
  static_assert(NB == 1 || NB == 2, "one or two rows of X");
  using D = Decode<BITS>;
  __shared__ uint32_t xq_lds[NB][SPL][kSeg / 2][64];   // pair j of segment lane + 64 t, X row b
  __shared__ float xs_lds[NB][SPL][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nseg = (n + kSeg - 1) / kSeg;
  const uint32_t ones = 0x3C003C00u;  // (1.0, 1.0) in float16
  // Wave w forms slots u = w, w + 4, ... of (X row, segment slot) pairs.
  for (int u = wave; u < NB * SPL; u += kWaves) {
    const int b = u / SPL, t = u % SPL;
    const int k0 = (lane + 64 * t) * kSeg;
    uint32_t xn[kSeg / 2];
    if (k0 + kSeg <= n) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(X + (int64_t)b * ldx + k0 + 8 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) xn[4 * v + e] = q[e];
      }
    } else {
#pragma unroll
      for (int v = 0; v < kSeg / 2; ++v) xn[v] = 0u;
    }
    float xs = 0.f;
#pragma unroll
    for (int j = 0; j < kSeg / 2; ++j) {
      xq_lds[b][t][j][lane] = x_pair(xn, D::first(j), D::H);
      xs = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, xn[j]), __builtin_bit_cast(half2_t, ones), xs, false);
    }
    xs_lds[b][t][lane] = xs;
  }
  __syncthreads();
  int gs[SPL];
#pragma unroll
  for (int t = 0; t < SPL; ++t) gs[t] = group_size > 0 ? min(lane + 64 * t, nseg - 1) * kSeg / group_size : 0;
  // A row's words and grid values for this lane's segments, with no branch
  // (every segment is whole; a lane past the last segment reads the last one
  // and row_out leaves it out), so the waits for one row's loads never wait
  // for the next row's.
  auto load_row = [&](int r, uint32_t (&w)[SPL][BITS], float (&sv)[SPL], float (&zv)[SPL]) {
#pragma unroll
    for (int t = 0; t < SPL; ++t) {
      const int seg = min(lane + 64 * t, nseg - 1);
      const uint32_t* wr = packed + (int64_t)r * ldp + (int64_t)seg * BITS;
      if constexpr (BITS == 4) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr));
#pragma unroll
        for (int e = 0; e < 4; ++e) w[t][e] = q[e];
      } else {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 q = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(wr));
        w[t][0] = q[0];
        w[t][1] = q[1];
      }
      sv[t] = scales[(int64_t)r * G + gs[t]];
      zv[t] = (float)zeros[(int64_t)r * G + gs[t]];
    }
  };
  auto row_out = [&](int r, const uint32_t (&w)[SPL][BITS], const float (&sv)[SPL], const float (&zv)[SPL]) {
    float yacc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) yacc[b] = 0.f;
#pragma unroll
    for (int t = 0; t < SPL; ++t) {
      if (lane + 64 * t < nseg) {
        uint32_t pr[kSeg / 2];
        D::pairs(w[t], pr);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < kSeg / 2; ++j)
            a = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pr[j]),
                                       __builtin_bit_cast(half2_t, xq_lds[b][t][j][lane]), a, false);
          yacc[b] = __builtin_fmaf(sv[t], __builtin_fmaf(a, kTwo24, -zv[t] * xs_lds[b][t][lane]), yacc[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = wave_sum(yacc[b]);
      if (lane == 0) Y[(int64_t)b * ldy + r] = v;
    }
  };
  const int nwv = (int)gridDim.x * kWaves;
  uint32_t w0[SPL][BITS], w1[SPL][BITS];
  float s0[SPL], z0[SPL], s1[SPL], z1[SPL];
  int r = (int)blockIdx.x * kWaves + wave;
  if (r < m) load_row(r, w0, s0, z0);
  for (; r < m; r += 2 * nwv) {
    const int r1 = r + nwv;
    if (r1 < m) load_row(r1, w1, s1, z1);
    row_out(r, w0, s0, z0);
    if (r1 < m) {
      if (r1 + nwv < m) load_row(r1 + nwv, w0, s0, z0);
      row_out(r1, w1, s1, z1);
    }
  }
}

// Matrix-core path (any batch, per-row grids or contiguous groups of a
// multiple of 128 columns, no g_idx).  The same subnormal code pairs are the
// A operand of v_mfma_f32_16x16x32_f16 (A element (row l%16, k 8*(l/16) + e),
// B element (k 8*(l/16) + e, column l%16), accumulator register i of lane l:
// row 4*(l/16) + i, column l%16 — checked with an in-bounds probe).  A chunk
// is 128 columns: lane quarter q takes segment 4*chunk + q, and MFMA j of the
// chunk takes the segment's code pairs 4j .. 4j+3 (8 columns per quarter), so
// a chunk never straddles a group.  sum x per column comes from one more MFMA
// with all-ones subnormal codes.  At the end of each group:
//   y += s * (2^24 * acc - z * 2^24 * acc_ones).
// A workgroup owns 16*RT rows and 16*NT columns of Y (batch rows of X); its
// four waves split the chunks and add their partial sums through LDS in a
// fixed order.  The next chunk's words and X are loaded while the current one
// multiplies.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ inline half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

template <int BITS, int RT, int NT>
__global__ __launch_bounds__(kThreads) void dequant_mfma_kernel(
    const uint32_t* __restrict__ packed, int m, int n, int64_t ldp, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int G, int group_size, const uint16_t* __restrict__ X, int batch,
    int64_t ldx, float* __restrict__ Y, int64_t ldy, int vec_w, int vec_x) {
  using D = Decode<BITS>;
  __shared__ floatx4 red[kWaves - 1][RT][NT][64];
  const int lane = threadIdx.x & 63, q = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r0 = (int)blockIdx.x * 16 * RT;
  const int c0 = (int)blockIdx.y * 16 * NT;
  const int nseg = (n + kSeg - 1) / kSeg;
  const int nw = (int)(((int64_t)n * BITS + 31) / 32);
  const int nchunk = (nseg + 3) / 4;
  const int gchunks = group_size > 0 ? group_size / 128 : nchunk;
  // The workgroup's waves share the rows and split the chunks (columns).
  const int c_lo = wave * nchunk / kWaves, c_hi = (wave + 1) * nchunk / kWaves;
  floatx4 acc[RT][NT], accx[NT], yacc[RT][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    accx[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = yacc[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const half8_t ones = as_half8(0x00010001u, 0x00010001u, 0x00010001u, 0x00010001u);
  // Operands of one chunk as loaded: row words and natural X pairs.
  struct Raw {
    uint32_t w[RT][BITS];
    uint32_t xn[NT][kSeg / 2];
  };
  auto load = [&](Raw& o, int ch) {
    const int seg = 4 * ch + q;
    const int k0 = seg * kSeg;
    const bool whole = k0 + kSeg <= n;  // implies seg < nseg
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = r0 + 16 * rt + c16;
      const uint32_t* wr = packed + (int64_t)(row < m ? row : r0) * ldp + (int64_t)seg * BITS;
      if (row < m && whole && vec_w && BITS == 4) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr));
#pragma unroll
        for (int e = 0; e < BITS; ++e) o.w[rt][e] = t[e & 3];
      } else {
#pragma unroll
        for (int e = 0; e < BITS; ++e)
          o.w[rt][e] = (row < m && seg < nseg && seg * BITS + e < nw) ? __builtin_nontemporal_load(wr + e) : 0u;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // Every lane loads (from row min(b, batch-1)) so the wave does not
      // branch on the batch; rows past the batch are zeroed afterwards.
      const int b = c0 + 16 * nt + c16;
      const uint32_t keep = b < batch ? 0xFFFFFFFFu : 0u;
      const uint16_t* xr = X + (int64_t)(b < batch ? b : batch - 1) * ldx + k0;
      if (whole && vec_x) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(xr + 8 * v);
#pragma unroll
          for (int e = 0; e < 4; ++e) o.xn[nt][4 * v + e] = t[e] & keep;
        }
      } else {
#pragma unroll
        for (int t = 0; t < kSeg / 2; ++t) {
          const uint32_t lo = k0 + 2 * t < n ? xr[2 * t] : 0u;
          const uint32_t hi = k0 + 2 * t + 1 < n ? xr[2 * t + 1] : 0u;
          o.xn[nt][t] = (lo | (hi << 16)) & keep;
        }
      }
    }
  };
  auto compute = [&](const Raw& cur, int ch) {
    half8_t bop[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bop[nt][j] = as_half8(x_pair(cur.xn[nt], D::first(4 * j), D::H), x_pair(cur.xn[nt], D::first(4 * j + 1), D::H),
                              x_pair(cur.xn[nt], D::first(4 * j + 2), D::H), x_pair(cur.xn[nt], D::first(4 * j + 3), D::H));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t p[kSeg / 2];
      D::pairs(cur.w[rt], p);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t aop = as_half8(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[nt][j], acc[rt][nt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) accx[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, bop[nt][j], accx[nt], 0, 0, 0);
    if ((ch + 1) % gchunks == 0 || ch + 1 == c_hi) {
      const int g = group_size > 0 ? ch / gchunks : 0;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = r0 + 16 * rt + 4 * q + i;
          const float sc = row < m ? scales[(int64_t)row * G + g] : 0.f;
          const float z = row < m ? (float)zeros[(int64_t)row * G + g] : 0.f;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            yacc[rt][nt][i] = __builtin_fmaf(sc, __builtin_fmaf(acc[rt][nt][i], kTwo24, -z * (accx[nt][i] * kTwo24)),
                                             yacc[rt][nt][i]);
        }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        accx[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // Two named buffers (a runtime index into an array of them would put the
  // operands in scratch memory): the next chunk loads while one multiplies.
  Raw b0, b1;
  if (c_lo < c_hi) load(b0, c_lo);
  for (int ch = c_lo; ch < c_hi; ch += 2) {
    if (ch + 1 < c_hi) load(b1, ch + 1);
    compute(b0, ch);
    if (ch + 1 < c_hi) {
      if (ch + 2 < c_hi) load(b0, ch + 2);
      compute(b1, ch + 1);
    }
  }
  // Partial sums of waves 1..3 through LDS; wave 0 adds them in wave order.
  if (wave > 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red[wave - 1][rt][nt][lane] = yacc[rt][nt];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 v = yacc[rt][nt];
#pragma unroll
      for (int w = 0; w < kWaves - 1; ++w) v += red[w][rt][nt][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + 16 * rt + 4 * q + i, col = c0 + 16 * nt + c16;
        if (row < m && col < batch) Y[(int64_t)col * ldy + row] = v[i];
      }
    }
}

// Decode batches of 3 to 16 rows of X on large layers (per-row grids, 2- or
// 4-bit, n a multiple of 32): the kernel above reads X once per wave and
// chunk, as many bytes as the weights it multiplies.  Here the workgroup
// stages X once for all its rows, in panels of kStreamChunks chunks, already
// in B-operand order (xs[chunk][j][q][b] = the 8 values MFMA j of lane
// quarter q takes for X row b) with each segment's sum beside it, double
// buffered so the next panel is staged while this one multiplies (one
// barrier per panel).  Each wave owns TPW tiles of 16 rows for the whole of
// n: per chunk it reads the B operands once from LDS and multiplies every
// tile's decoded codes into that tile's accumulator; the words of the next
// panel are loaded while the current one multiplies.  The z term uses the
// staged segment sums (sum x over the row), so no all-ones MFMA is needed.
constexpr int kStreamChunks = 4;  // chunks (128 columns each) per X panel
constexpr int kStreamMaxTpw = 3;   // tiles of 16 rows per wave at most
constexpr int kStreamMinTiles = 1024;  // 16-row tiles a layer needs for this kernel (a wave per SIMD)
constexpr int kStreamGroupMinTiles = 768;  // the same for contiguous groups

template <int BITS> struct SegWords;
template <> struct SegWords<4> { typedef u32x4 type; };
template <> struct SegWords<2> { typedef unsigned int type __attribute__((ext_vector_type(2))); };

template <int BITS, int NB, int TPW, bool GROUPED>
__global__ __launch_bounds__(kThreads) void dequant_mfma_stream_kernel(
    const uint32_t* __restrict__ packed, int m, int n, int64_t ldp, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int G, int gchunks, const uint16_t* __restrict__ X, int batch, int64_t ldx,
    float* __restrict__ Y, int64_t ldy) {
  static_assert(BITS == 2 || BITS == 4, "whole-word segments");
  static_assert(NB == 4 || NB == 8 || NB == 16, "X rows staged");
  using D = Decode<BITS>;
  using WordT = typename SegWords<BITS>::type;
  constexpr int PC = kStreamChunks;
  constexpr int kUnits = NB * PC * 4;  // staged (X row, segment) pairs per panel
  static_assert(kUnits % 64 == 0 && kUnits <= kThreads, "whole waves stage");
  __shared__ u32x4 xs[2][PC][4][4][NB];
  __shared__ floatx4 xsum[2][PC][NB];
  // Groups (GROUPED): (s, z) of the workgroup's rows for each chunk's group,
  // panel p in buffer p mod 3: while panel p multiplies, a wave still folds
  // panel p - 1's last chunk and a faster wave may already store panel p + 1,
  // so three panels are live at once.
  constexpr int kWgRows = kWaves * TPW * 16;
  __shared__ float2 gsz[GROUPED ? 3 : 1][GROUPED ? PC : 1][GROUPED ? kWgRows : 1];
  const int lane = threadIdx.x & 63, q = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nseg = n / kSeg;
  const int nchunk = (nseg + 3) / 4;
  const int npanel = (nchunk + PC - 1) / PC;
  const int bb = c16 < batch ? c16 : batch - 1;  // X row this lane's B operands come from
  const int tile0 = (int)blockIdx.x * kWaves * TPW + wave;
  const uint32_t* wrow[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int row = (tile0 + kWaves * i) * 16 + c16;
    wrow[i] = packed + (int64_t)(row < m ? row : m - 1) * ldp;
  }
  // Staging: thread u < kUnits takes X row b = u / (4 PC) and panel segment
  // u % (4 PC), so neighbouring threads read neighbouring 64-byte pieces.
  const int su = threadIdx.x;
  const int sb = su / (4 * PC), sseg = su % (4 * PC);
  const uint16_t* xrow = X + (int64_t)(sb < batch ? sb : batch - 1) * ldx;
  auto stage_load = [&](u32x4 (&xr)[4], int p) {
    const int seg = p * 4 * PC + sseg;
    const int s = seg < nseg ? seg : nseg - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(xrow + (int64_t)s * kSeg);
#pragma unroll
    for (int v = 0; v < 4; ++v) xr[v] = seg < nseg ? src[v] : u32x4{0u, 0u, 0u, 0u};
  };
  auto stage_store = [&](const u32x4 (&xr)[4], int buf) {
    uint32_t xn[kSeg / 2];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) xn[4 * v + e] = xr[v][e];
    const int c = sseg >> 2, qs = sseg & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xs[buf][c][j][qs][sb] = u32x4{x_pair(xn, D::first(4 * j), D::H), x_pair(xn, D::first(4 * j + 1), D::H),
                                    x_pair(xn, D::first(4 * j + 2), D::H), x_pair(xn, D::first(4 * j + 3), D::H)};
    const uint32_t ones = 0x3C003C00u;  // (1.0, 1.0) in float16
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kSeg / 2; ++j)
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, xn[j]), __builtin_bit_cast(half2_t, ones), s, false);
    xsum[buf][c][sb][qs] = s;
  };
  // Grid values of a panel (GROUPED): thread t < kWgRows stages its row's
  // (s, z) for the panel's chunks (neighbouring groups of one row share a
  // cache line); the loads have no branch (threads past kWgRows and rows
  // past m read a clamped row, groups past G the last one).
  static_assert(kWgRows <= kThreads, "one thread per workgroup row");
  const int wg_row0 = (int)blockIdx.x * kWgRows;
  const int sz_row = min(wg_row0 + min((int)threadIdx.x, kWgRows - 1), m - 1);
  auto sz_load = [&](float2 (&v)[PC], int p) {
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      const int gi = min((p * PC + c) / gchunks, G - 1);
      v[c] = float2{scales[(int64_t)sz_row * G + gi], (float)zeros[(int64_t)sz_row * G + gi]};
    }
  };
  auto sz_store = [&](const float2 (&v)[PC], int buf) {
    if ((int)threadIdx.x < kWgRows) {
#pragma unroll
      for (int c = 0; c < PC; ++c) gsz[buf][c][threadIdx.x] = v[c];
    }
  };
  // A panel's words for the wave's tiles: segment 4 (p PC + c) + q of each
  // tile row, clamped to the last segment (its X is staged as zeros).
  struct Words {
    WordT w[TPW][PC];
  };
  auto load_words = [&](Words& o, int p) {
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      const int seg = min(4 * (p * PC + c) + q, nseg - 1);
#pragma unroll
      for (int i = 0; i < TPW; ++i)
        o.w[i][c] = __builtin_nontemporal_load(reinterpret_cast<const WordT*>(wrow[i] + (int64_t)seg * BITS));
    }
  };
  // Per-row grids: one accumulator per tile over all of n and sum x over
  // the row.  Groups: every chunk is folded into y on its own (the fold is
  // linear, so a group of several chunks is the sum of its chunks' folds),
  // one chunk late: chunk c accumulates into accs[c & 1] and its fold waits
  // until chunk c + 1's products are issued, so it never waits for the
  // matrix core.
  floatx4 accs[GROUPED ? 2 : 1][TPW];
#pragma unroll
  for (int k = 0; k < (GROUPED ? 2 : 1); ++k)
#pragma unroll
    for (int i = 0; i < TPW; ++i) accs[k][i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float sx = 0.f;
  float sxc[2] = {0.f, 0.f};
  floatx4 yacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) yacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  // y += s (2^24 acc - z sum x) for the chunk held in accs[par] (chunk fc of
  // the panel whose (s, z) are in gsz[fbuf]), then that accumulator starts
  // afresh.
  auto fold = [&](int par, int fbuf, int fc) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 v = gsz[fbuf][fc][(wave + kWaves * i) * 16 + 4 * q + e];
        yacc[i][e] = __builtin_fmaf(v.x, __builtin_fmaf(accs[par][i][e], kTwo24, -v.y * sxc[par]), yacc[i][e]);
      }
      accs[par][i] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto compute = [&](const Words& o, int buf, int p) {
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      const int par = GROUPED ? (c & 1) : 0;
      half8_t bop[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bop[j] = __builtin_bit_cast(half8_t, xs[buf][c][j][q][bb]);
      const floatx4 s4 = xsum[buf][c][bb];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        uint32_t w[BITS];
#pragma unroll
        for (int e = 0; e < BITS; ++e) w[e] = o.w[i][c][e];
        uint32_t pr[kSeg / 2];
        D::pairs(w, pr);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          accs[par][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              as_half8(pr[4 * j], pr[4 * j + 1], pr[4 * j + 2], pr[4 * j + 3]), bop[j], accs[par][i], 0, 0, 0);
      }
      if constexpr (GROUPED) {
        float t = s4[0];
        t += s4[1];
        t += s4[2];
        t += s4[3];
        sxc[par] = t;
        // the previous chunk: c - 1 of this panel, or the last chunk of the
        // previous panel
        if (c > 0)
          fold(par ^ 1, p % 3, c - 1);
        else if (p > 0)
          fold(par ^ 1, (p + 2) % 3, PC - 1);
      } else {
        sx += s4[0];
        sx += s4[1];
        sx += s4[2];
        sx += s4[3];
      }
    }
  };
  // Panel 0 staged before the loop; panel p + 1's X and words load while
  // panel p multiplies.  Two named word buffers (a runtime index into an
  // array of them would put them in scratch memory).
  Words wa, wb;
  u32x4 xr[4];
  float2 szr[PC];
  if (su < kUnits) {
    stage_load(xr, 0);
    stage_store(xr, 0);
  }
  if constexpr (GROUPED) {
    sz_load(szr, 0);
    sz_store(szr, 0);
  }
  load_words(wa, 0);
  __syncthreads();
  for (int p = 0; p < npanel; p += 2) {
    const bool more1 = p + 1 < npanel;
    if (more1) {
      if (su < kUnits) stage_load(xr, p + 1);
      if constexpr (GROUPED) sz_load(szr, p + 1);
      load_words(wb, p + 1);
    }
    compute(wa, 0, p);
    if (more1 && su < kUnits) stage_store(xr, 1);
    if constexpr (GROUPED) {
      if (more1) sz_store(szr, (p + 1) % 3);
    }
    __syncthreads();
    if (!more1) break;
    const bool more2 = p + 2 < npanel;
    if (more2) {
      if (su < kUnits) stage_load(xr, p + 2);
      if constexpr (GROUPED) sz_load(szr, p + 2);
      load_words(wa, p + 2);
    }
    compute(wb, 1, p + 1);
    if (more2 && su < kUnits) stage_store(xr, 0);
    if constexpr (GROUPED) {
      if (more2) sz_store(szr, (p + 2) % 3);
    }
    __syncthreads();
  }
  if constexpr (GROUPED) fold((PC - 1) & 1, (npanel - 1) % 3, PC - 1);
  // Per-row grids: y = s (2^24 acc - z sum x); groups: the folded sums.
  // Rows past m and X rows past the batch are not stored.
  if (c16 >= batch) return;
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = (tile0 + kWaves * i) * 16 + 4 * q + e;
      if (row < m) {
        if constexpr (GROUPED) {
          Y[(int64_t)c16 * ldy + row] = yacc[i][e];
        } else {
          const float sc = scales[(int64_t)row * G];
          const float z = (float)zeros[(int64_t)row * G];
          Y[(int64_t)c16 * ldy + row] = sc * __builtin_fmaf(accs[0][i][e], kTwo24, -z * sx);
        }
      }
    }
}

// Prefill-sized batches: a workgroup owns 128 rows of W x 128 rows of X
// (4 waves as 2 x 2, each 64 x 64 = 4 x 4 MFMA tiles).  Per 128-column chunk
// the X tile is staged once in LDS, already in code-pair order
// (Xs[b][segment][pair] = (x_a, x_{a+H}) as in x_pair), so each MFMA B
// operand is one 16-byte LDS read; the codes are decoded straight into A
// registers as in the kernel above; the next chunk's X and codes are loaded
// into registers while the current chunk multiplies.
constexpr int kPM = 128, kPN = 128;

template <int BITS>
__global__ __launch_bounds__(kThreads) void dequant_gemm_lds_kernel(
    const uint32_t* __restrict__ packed, int m, int n, int64_t ldp, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int G, int group_size, const uint16_t* __restrict__ X, int batch,
    int64_t ldx, float* __restrict__ Y, int64_t ldy, int vec_w, int vec_x) {
  using D = Decode<BITS>;
  __shared__ __attribute__((aligned(16))) uint32_t Xs[2][kPN][4][kSeg / 2];
  __shared__ __attribute__((aligned(16))) float Xsum[2][kPN][4];   // sum of each staged segment
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int r0 = (int)blockIdx.x * kPM + wr * 64;   // this wave's first row
  const int b0 = (int)blockIdx.y * kPN;             // the workgroup's first X row
  const int nseg = (n + kSeg - 1) / kSeg;
  const int nw = (int)(((int64_t)n * BITS + 31) / 32);
  const int nchunk = (nseg + 3) / 4;
  const int gchunks = group_size > 0 ? group_size / 128 : nchunk;
  floatx4 acc[4][4], yacc[4][4];
  float xsg[4];   // sum of X over the current group's columns, for X row of column tile nt
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    xsg[nt] = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt][nt] = yacc[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  // X staging: thread t handles (X row t/2, segments 2*(t%2), 2*(t%2)+1) of the tile.
  const int xb = tid >> 1, xs0 = 2 * (tid & 1);
  struct Raw {
    uint32_t xn[2][kSeg / 2];
    uint32_t w[4][BITS];
  };
  auto load = [&](Raw& o, int ch) {
    const int brow = b0 + xb;
    const uint32_t keep = brow < batch ? 0xFFFFFFFFu : 0u;
    const uint16_t* xr = X + (int64_t)(brow < batch ? brow : batch - 1) * ldx;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k0 = (4 * ch + xs0 + u) * kSeg;
      if (k0 + kSeg <= n && vec_x) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(xr + k0 + 8 * v);
#pragma unroll
          for (int e = 0; e < 4; ++e) o.xn[u][4 * v + e] = t[e] & keep;
        }
      } else {
#pragma unroll
        for (int t = 0; t < kSeg / 2; ++t) {
          const uint32_t lo = k0 + 2 * t < n ? xr[k0 + 2 * t] : 0u;
          const uint32_t hi = k0 + 2 * t + 1 < n ? xr[k0 + 2 * t + 1] : 0u;
          o.xn[u][t] = (lo | (hi << 16)) & keep;
        }
      }
    }
    const int seg = 4 * ch + q;
    const bool whole = (seg + 1) * kSeg <= n;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int row = r0 + 16 * rt + c16;
      const uint32_t* wr_ = packed + (int64_t)(row < m ? row : 0) * ldp + (int64_t)seg * BITS;
      if (row < m && whole && vec_w && BITS == 4) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr_));
#pragma unroll
        for (int e = 0; e < BITS; ++e) o.w[rt][e] = t[e & 3];
      } else {
#pragma unroll
        for (int e = 0; e < BITS; ++e)
          o.w[rt][e] = (row < m && seg < nseg && seg * BITS + e < nw) ? __builtin_nontemporal_load(wr_ + e) : 0u;
      }
    }
  };
  auto stage = [&](const Raw& o, int buf) {
    const uint32_t one2 = 0x3C003C00u;  // (1.0, 1.0) in float16
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float sx = 0.f;
#pragma unroll
      for (int j = 0; j < kSeg / 2; j += 4) {
        const u32x4 v = {x_pair(o.xn[u], D::first(j), D::H), x_pair(o.xn[u], D::first(j + 1), D::H),
                         x_pair(o.xn[u], D::first(j + 2), D::H), x_pair(o.xn[u], D::first(j + 3), D::H)};
        *reinterpret_cast<u32x4*>(&Xs[buf][xb][xs0 + u][j]) = v;
      }
#pragma unroll
      for (int t = 0; t < kSeg / 2; ++t)
        sx = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, o.xn[u][t]), __builtin_bit_cast(half2_t, one2), sx,
                                    false);
      Xsum[buf][xb][xs0 + u] = sx;
    }
  };
  auto compute = [&](const Raw& o, int buf, int ch) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const floatx4 sv = *reinterpret_cast<const floatx4*>(&Xsum[buf][wc * 64 + 16 * nt + c16][0]);
      xsg[nt] += (sv[0] + sv[1]) + (sv[2] + sv[3]);
    }
    // MFMA step j: the four B operands, then each row tile's four code pairs.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t bop[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&Xs[buf][wc * 64 + 16 * nt + c16][q][4 * j]);
        bop[nt] = as_half8(v[0], v[1], v[2], v[3]);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const half8_t aop = as_half8(D::pair(o.w[rt], 4 * j), D::pair(o.w[rt], 4 * j + 1),
                                     D::pair(o.w[rt], 4 * j + 2), D::pair(o.w[rt], 4 * j + 3));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[nt], acc[rt][nt], 0, 0, 0);
      }
    }
    if ((ch + 1) % gchunks == 0 || ch + 1 == nchunk) {
      const int g = group_size > 0 ? ch / gchunks : 0;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = r0 + 16 * rt + 4 * q + i;
          const float sc = row < m ? scales[(int64_t)row * G + g] : 0.f;
          const float szc = sc * (row < m ? (float)zeros[(int64_t)row * G + g] : 0.f);
          const float s24 = sc * kTwo24;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            yacc[rt][nt][i] = __builtin_fmaf(s24, acc[rt][nt][i], __builtin_fmaf(-szc, xsg[nt], yacc[rt][nt][i]));
        }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        xsg[nt] = 0.f;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // Two named register buffers (see the kernel above) and two LDS buffers.
  Raw ra, rb;
  load(ra, 0);
  stage(ra, 0);
  __syncthreads();
  for (int ch = 0; ch < nchunk; ch += 2) {
    if (ch + 1 < nchunk) load(rb, ch + 1);
    compute(ra, 0, ch);
    if (ch + 1 < nchunk) {
      stage(rb, 1);           // buffer 1 was last read before the previous barrier
      __syncthreads();
      if (ch + 2 < nchunk) load(ra, ch + 2);
      compute(rb, 1, ch + 1);
      if (ch + 2 < nchunk) stage(ra, 0);
      __syncthreads();
    }
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + 16 * rt + 4 * q + i, col = b0 + wc * 64 + 16 * nt + c16;
        if (row < m && col < batch) Y[(int64_t)col * ldy + row] = yacc[rt][nt][i];
      }
}

template <int BITS, int RT, int NT>
void launch_mfma(hipStream_t st, const uint32_t* packed, int m, int n, int64_t ldp, const float* scales,
                 const uint8_t* zeros, int G, int group_size, const uint16_t* X, int batch, int64_t ldx, float* Y,
                 int64_t ldy, int vec_w, int vec_x) {
  const dim3 grid((unsigned)ceil_div(m, (int64_t)16 * RT), (unsigned)ceil_div(batch, (int64_t)16 * NT));
  dequant_mfma_kernel<BITS, RT, NT><<<grid, kThreads, 0, st>>>(packed, m, n, ldp, scales, zeros, G, group_size, X,
                                                               batch, ldx, Y, ldy, vec_w, vec_x);
}

// The streaming kernel with `tpw` tiles of 16 rows per wave.
template <int BITS, int NB, bool GROUPED>
void launch_stream_grouped(hipStream_t st, unsigned grid, int tpw, const uint32_t* packed, int m, int n,
                           int64_t ldp, const float* scales, const uint8_t* zeros, int G, int gchunks,
                           const uint16_t* X, int batch, int64_t ldx, float* Y, int64_t ldy) {
  if (tpw >= 3)
    dequant_mfma_stream_kernel<BITS, NB, 3, GROUPED><<<grid, kThreads, 0, st>>>(packed, m, n, ldp, scales, zeros, G,
                                                                               gchunks, X, batch, ldx, Y, ldy);
  else if (tpw == 2)
    dequant_mfma_stream_kernel<BITS, NB, 2, GROUPED><<<grid, kThreads, 0, st>>>(packed, m, n, ldp, scales, zeros, G,
                                                                               gchunks, X, batch, ldx, Y, ldy);
  else
    dequant_mfma_stream_kernel<BITS, NB, 1, GROUPED><<<grid, kThreads, 0, st>>>(packed, m, n, ldp, scales, zeros, G,
                                                                               gchunks, X, batch, ldx, Y, ldy);
}

// Tiles per wave of the streaming kernel: the most (up to kStreamMaxTpw) that
// still give every CU a workgroup.  With four staged rows of X, one tile per
// wave (three times the workgroups, each staging X again) keeps more loads in
// flight and is faster; with eight or sixteen the staging costs more than
// that gains (49152 x 12288 4-bit: batch 3 73 vs 82 us, batch 16 92 vs 86 us).
template <int BITS, int NB>
void launch_stream_nb(hipStream_t st, const uint32_t* packed, int m, int n, int64_t ldp, const float* scales,
                      const uint8_t* zeros, int G, int group_size, const uint16_t* X, int batch, int64_t ldx,
                      float* Y, int64_t ldy, int64_t tiles) {
  int tpw = NB == 4 ? 1 : kStreamMaxTpw;
  while (tpw > 1 && ceil_div(tiles, (int64_t)kWaves * tpw) < kStreamMinTiles / kWaves) --tpw;
  const unsigned grid = (unsigned)ceil_div(tiles, (int64_t)kWaves * tpw);
  if (group_size > 0)
    launch_stream_grouped<BITS, NB, true>(st, grid, tpw, packed, m, n, ldp, scales, zeros, G, group_size / 128, X,
                                          batch, ldx, Y, ldy);
  else
    launch_stream_grouped<BITS, NB, false>(st, grid, tpw, packed, m, n, ldp, scales, zeros, G, 1, X, batch, ldx, Y,
                                           ldy);
}

template <int BITS>
void launch_stream(hipStream_t st, const uint32_t* packed, int m, int n, int64_t ldp, const float* scales,
                   const uint8_t* zeros, int G, int group_size, const uint16_t* X, int batch, int64_t ldx, float* Y,
                   int64_t ldy, int64_t tiles) {
  if (batch <= 4)
    launch_stream_nb<BITS, 4>(st, packed, m, n, ldp, scales, zeros, G, group_size, X, batch, ldx, Y, ldy, tiles);
  else if (batch <= 8)
    launch_stream_nb<BITS, 8>(st, packed, m, n, ldp, scales, zeros, G, group_size, X, batch, ldx, Y, ldy, tiles);
  else
    launch_stream_nb<BITS, 16>(st, packed, m, n, ldp, scales, zeros, G, group_size, X, batch, ldx, Y, ldy, tiles);
}

template <int BITS>
void launch_mfma_shape(hipStream_t st, const uint32_t* packed, int m, int n, int64_t ldp, const float* scales,
                       const uint8_t* zeros, int G, int group_size, const uint16_t* X, int batch, int64_t ldx,
                       float* Y, int64_t ldy, int vec_w, int vec_x) {
  // Decode-sized batches: one 16-column tile, 16 or 64 rows per workgroup
  // (more workgroups for short layers); up to 64 rows of X: that kernel once
  // per 16 rows (it streams the weights at near-HBM rate, the 128-wide tile
  // below would spend most of its work on padding); larger batches: 128 x 128
  // tiles with X staged in LDS.
  if (batch <= 64) {
    // The streaming kernel on layers of at least kStreamMinTiles tiles; on
    // layers of 3/4 of that only for more than eight rows of X (12288 x
    // 49152: batch 3-8 102-123 us on the kernel below against 142-152 us,
    // batch 12-16 160-203 us against 149 us).
    const int64_t tiles = ceil_div(m, (int64_t)16);
    const bool stream_layout = BITS != 3 && n >= kSeg && n % kSeg == 0 && vec_w && vec_x;
    for (int b0 = 0; b0 < batch; b0 += 16) {
      const int cb = std::min(16, batch - b0);
      const uint16_t* Xc = X + (int64_t)b0 * ldx;
      float* Yc = Y + (int64_t)b0 * ldy;
      const bool stream = stream_layout && (tiles >= (int64_t)kStreamMinTiles ||
                                            (tiles >= (int64_t)kStreamMinTiles * 3 / 4 && cb > 8) ||
                                            (group_size > 0 && tiles >= (int64_t)kStreamGroupMinTiles));
      if constexpr (BITS != 3) {
        if (stream) {
          launch_stream<BITS>(st, packed, m, n, ldp, scales, zeros, G, group_size, Xc, cb, ldx, Yc, ldy, tiles);
          continue;
        }
      }
      if (m <= 16384)
        launch_mfma<BITS, 1, 1>(st, packed, m, n, ldp, scales, zeros, G, group_size, Xc, cb, ldx, Yc, ldy, vec_w,
                                vec_x);
      else
        launch_mfma<BITS, 4, 1>(st, packed, m, n, ldp, scales, zeros, G, group_size, Xc, cb, ldx, Yc, ldy, vec_w,
                                vec_x);
    }
  } else {
    const dim3 grid((unsigned)ceil_div(m, (int64_t)kPM), (unsigned)ceil_div(batch, (int64_t)kPN));
    dequant_gemm_lds_kernel<BITS><<<grid, kThreads, 0, st>>>(packed, m, n, ldp, scales, zeros, G, group_size, X,
                                                             batch, ldx, Y, ldy, vec_w, vec_x);
  }
}

template <int BITS, int NB, bool PC>
void launch_nb(size_t shm_per_row, hipStream_t st, const uint32_t* packed, int m, int n, int64_t ldp,
               const float* scales, const uint8_t* zeros, int G, int group_size, const int32_t* g_idx,
               const uint16_t* X, int batch, int64_t ldx, float* Y, int64_t ldy, int vec_w, int vec_x) {
  constexpr int rows = rows_per_wave<NB>();
  // Waves loop over groups of `rows` rows; at most kGridCap workgroups.
  const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(m, (int64_t)rows * kWaves), kGridCap);
  // Per-code path: each wave stages its rows' (s, s*z) in LDS when they fit.
  const size_t need = shm_per_row * rows * kWaves;
  const size_t shm = PC && need <= kMaxStageBytes ? need : 0;
  dequant_gemv_kernel<BITS, NB, PC><<<grid, kThreads, shm, st>>>(packed, m, n, ldp, scales, zeros, G, group_size,
                                                                 g_idx, X, batch, ldx, Y, ldy, vec_w, vec_x, shm > 0);
}

template <int BITS, bool PC>
void launch_bits(size_t shm, hipStream_t st, const uint32_t* packed, int m, int n, int64_t ldp,
                 const float* scales, const uint8_t* zeros, int G, int group_size, const int32_t* g_idx,
                 const uint16_t* X, int batch, int64_t ldx, float* Y, int64_t ldy, int vec_w, int vec_x) {
  if (batch == 1)
    launch_nb<BITS, 1, PC>(shm, st, packed, m, n, ldp, scales, zeros, G, group_size, g_idx, X, batch, ldx, Y, ldy,
                           vec_w, vec_x);
  else if (batch == 2)
    launch_nb<BITS, 2, PC>(shm, st, packed, m, n, ldp, scales, zeros, G, group_size, g_idx, X, batch, ldx, Y, ldy,
                           vec_w, vec_x);
  else if (batch <= 4)
    launch_nb<BITS, 4, PC>(shm, st, packed, m, n, ldp, scales, zeros, G, group_size, g_idx, X, batch, ldx, Y, ldy,
                           vec_w, vec_x);
  else
    launch_nb<BITS, 8, PC>(shm, st, packed, m, n, ldp, scales, zeros, G, group_size, g_idx, X, batch, ldx, Y, ldy,
                           vec_w, vec_x);
}

}  // namespace
}  // namespace gptq

using namespace gptq;

namespace {

// The VALU kernel over batch rows b0 .. b0+bn-1 (bn <= GPTQ_GEMV_MAX_BATCH).
gptq_status launch_valu_rows(hipStream_t st, const uint32_t* packed, int m, int n, int64_t ld_packed, int bits,
                             const float* scales, const uint8_t* zeros, int G, int group_size, const int32_t* g_idx,
                             const uint16_t* X, int bn, int64_t ldx, float* Y, int64_t ldy, int vec_w, int vec_x,
                             bool per_code) {
  const int spl = (int)ceil_div(ceil_div(n, kSeg), 64);
  if (bn <= 2 && !per_code && vec_w && vec_x && bits != 3 && n % kSeg == 0 && spl <= kXregMaxSpl) {
    const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(m, kWaves), kXregGrid);
#define GPTQ_XREG(B, S)                                                                                              \
  do {                                                                                                               \
    if (bn == 1)                                                                                                     \
      dequant_gemv_xreg_kernel<B, S, 1><<<grid, kThreads, 0, st>>>(packed, m, n, ld_packed, scales, zeros, G,       \
                                                                   group_size, X, ldx, Y, ldy);                     \
    else                                                                                                             \
      dequant_gemv_xreg_kernel<B, S, 2><<<grid, kThreads, 0, st>>>(packed, m, n, ld_packed, scales, zeros, G,       \
                                                                   group_size, X, ldx, Y, ldy);                     \
  } while (0)
#define GPTQ_XREG_BITS(B)          \
  do {                             \
    switch (spl) {                 \
      case 1: GPTQ_XREG(B, 1); break; \
      case 2: GPTQ_XREG(B, 2); break; \
      case 3: GPTQ_XREG(B, 3); break; \
      case 4: GPTQ_XREG(B, 4); break; \
      case 5: GPTQ_XREG(B, 5); break; \
      default: GPTQ_XREG(B, 6); break; \
    }                              \
  } while (0)
    if (bits == 2)
      GPTQ_XREG_BITS(2);
    else
      GPTQ_XREG_BITS(4);
#undef GPTQ_XREG_BITS
#undef GPTQ_XREG
    GPTQ_TRY_LAUNCH();
    return GPTQ_OK;
  }
  const size_t shm_per_row = (size_t)G * sizeof(float2);
#define GPTQ_GEMV_BITS(B)                                                                                      \
  do {                                                                                                         \
    if (per_code)                                                                                              \
      launch_bits<B, true>(shm_per_row, st, packed, m, n, ld_packed, scales, zeros, G, group_size, g_idx, X, bn, \
                           ldx, Y, ldy, vec_w, vec_x);                                                         \
    else                                                                                                       \
      launch_bits<B, false>(0, st, packed, m, n, ld_packed, scales, zeros, G, group_size, g_idx, X, bn, ldx, Y,  \
                            ldy, vec_w, vec_x);                                                                \
  } while (0)
  if (bits == 2)
    GPTQ_GEMV_BITS(2);
  else if (bits == 3)
    GPTQ_GEMV_BITS(3);
  else
    GPTQ_GEMV_BITS(4);
#undef GPTQ_GEMV_BITS
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

// Y = X W^T for any batch: the matrix-core kernel when the groups are
// contiguous multiples of 128 columns (or one per row) and the batch is at
// least min_mfma_batch, else the VALU kernel over chunks of
// GPTQ_GEMV_MAX_BATCH rows of X (act-order g_idx, narrower groups).
gptq_status dequant_product(const uint32_t* packed, int64_t m, int64_t n, int64_t ld_packed, int bits,
                            const float* scales, const uint8_t* zeros, int64_t G, int group_size,
                            const int32_t* g_idx, const uint16_t* X, int64_t batch, int64_t ldx, float* Y,
                            int64_t ldy, void* stream, int64_t min_mfma_batch) {
  if (m < 0 || n < 0 || group_size < 0 || G < 1 || batch < 0) return GPTQ_ERR_INVALID_ARG;
  if (!(bits == 2 || bits == 3 || bits == 4)) return GPTQ_ERR_INVALID_ARG;
  if (m > ((int64_t)1 << 31) - 1 || n > ((int64_t)1 << 30) || G > ((int64_t)1 << 30) ||
      ceil_div(batch, 128) > 65535)
    return GPTQ_ERR_UNSUPPORTED;
  if (m == 0 || batch == 0) return GPTQ_OK;
  if (ld_packed < ceil_div(n * bits, 32) || ldx < n || ldy < m) return GPTQ_ERR_INVALID_ARG;
  if (g_idx == nullptr && group_size > 0 && G < ceil_div(n, group_size)) return GPTQ_ERR_INVALID_ARG;
  if (Y == nullptr || (n > 0 && (packed == nullptr || scales == nullptr || zeros == nullptr || X == nullptr)))
    return GPTQ_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int vec_w = (reinterpret_cast<uintptr_t>(packed) % 16 == 0) && (ld_packed % 4 == 0);
  const int vec_x = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && (ldx % 8 == 0);
  const int mi = (int)m, ni = (int)n, Gi = (int)G;
  const bool per_code = g_idx != nullptr || (group_size > 0 && group_size % 32 != 0);
  if (!per_code && group_size % 128 == 0 && batch >= min_mfma_batch) {
    const int bi = (int)batch;
    if (bits == 2)
      launch_mfma_shape<2>(st, packed, mi, ni, ld_packed, scales, zeros, Gi, group_size, X, bi, ldx, Y, ldy, vec_w, vec_x);
    else if (bits == 3)
      launch_mfma_shape<3>(st, packed, mi, ni, ld_packed, scales, zeros, Gi, group_size, X, bi, ldx, Y, ldy, vec_w, vec_x);
    else
      launch_mfma_shape<4>(st, packed, mi, ni, ld_packed, scales, zeros, Gi, group_size, X, bi, ldx, Y, ldy, vec_w, vec_x);
    GPTQ_TRY_LAUNCH();
    return GPTQ_OK;
  }
  for (int64_t b0 = 0; b0 < batch; b0 += GPTQ_GEMV_MAX_BATCH) {
    const int bn = (int)std::min<int64_t>(GPTQ_GEMV_MAX_BATCH, batch - b0);
    const gptq_status rc = launch_valu_rows(st, packed, mi, ni, ld_packed, bits, scales, zeros, Gi, group_size, g_idx,
                                            X + b0 * ldx, bn, ldx, Y + b0 * ldy, ldy, vec_w, vec_x, per_code);
    if (rc != GPTQ_OK) return rc;
  }
  return GPTQ_OK;
}

}  // namespace

extern "C" gptq_status gptq_dequant_gemv(const uint32_t* packed, int64_t m, int64_t n, int64_t ld_packed, int bits,
                                         const float* scales, const uint8_t* zeros, int64_t G, int group_size,
                                         const int32_t* g_idx, const uint16_t* X, int64_t batch, int64_t ldx,
                                         float* Y, int64_t ldy, void* stream) {
  if (batch < 1) return GPTQ_ERR_INVALID_ARG;
  // From three rows of X on, the matrix-core kernel is faster (one dot2 per
  // code pair per X row makes the VALU kernel compute-bound).
  return dequant_product(packed, m, n, ld_packed, bits, scales, zeros, G, group_size, g_idx, X, batch, ldx, Y, ldy,
                         stream, 3);
}

extern "C" gptq_status gptq_dequant_gemm(const uint32_t* packed, int64_t m, int64_t n, int64_t ld_packed, int bits,
                                         const float* scales, const uint8_t* zeros, int64_t G, int group_size,
                                         const int32_t* g_idx, const uint16_t* X, int64_t batch, int64_t ldx,
                                         float* Y, int64_t ldy, void* stream) {
  return dequant_product(packed, m, n, ld_packed, bits, scales, zeros, G, group_size, g_idx, X, batch, ldx, Y, ldy,
                         stream, 1);
}
