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
// LDS is double buffered, the next stage is prefetched into registers while
// the current one is multiplied, and MFMA fragments are double buffered in
// registers (the next 16-token step is read while the MFMAs of this one run).
//
// Accuracy: one float32 MFMA accumulator covers at most 32768 tokens (a
// "split"); each split writes its tile to the workspace and the reduce
// kernel sums the splits in float64, scales by alpha, adds the old H and
// mirrors the upper triangle.
#include "common.h"
#include "hessian_internal.h"

#include <atomic>
#include <type_traits>

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

// Upper-triangle tile t -> (I, J), I <= J.  Tiles are numbered by
// super-blocks of kGroup x kGroup bands (super-blocks row-major, tiles
// row-major inside each), so that the ~32 consecutive tiles one XCD runs at a
// time touch about 12 bands instead of all of them and mostly hit its L2.
constexpr int kGroup = 8;
__device__ inline void tile_coords(int t, int nb, int& I, int& J) {
  const int ng = (nb + kGroup - 1) / kGroup;
  I = J = 0;
  for (int gi = 0; gi < ng; ++gi) {
    const int i0 = gi * kGroup, i1 = min(nb, i0 + kGroup);
    for (int gj = gi; gj < ng; ++gj) {
      const int j0 = gj * kGroup, j1 = min(nb, j0 + kGroup);
      if (gj > gi) {
        const int w = j1 - j0, cnt = (i1 - i0) * w;
        if (t < cnt) {
          I = i0 + t / w;
          J = j0 + t % w;
          return;
        }
        t -= cnt;
      } else {
        const int w = i1 - i0, cnt = w * (w + 1) / 2;
        if (t < cnt) {
          int i = i0;
          while (t >= i1 - i) {
            t -= i1 - i;
            ++i;
          }
          I = i;
          J = i + t;
          return;
        }
        t -= cnt;
      }
    }
  }
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

  u32x4 pre[2][2][8];   // [slot][band][token row]; slot 1 is unused in this variant

  // Feature chunks of this thread in the two bands; interior chunks of whole
  // stages take a branch-free path so that all 16 loads are in flight at once.
  const int f0a = I * kTile + fc * 8, f0b = J * kTile + fc * 8;
  const bool interior = vec_ok && f0a + 8 <= n && f0b + 8 <= n;
  const uint16_t* pa = X + f0a;
  const uint16_t* pb = X + f0b;

  auto gload = [&](u32x4 (&pr)[2][8], int64_t t0) {
    if (interior && t0 + kKt16 <= t_end) {
      const int64_t trow = t0 + tg * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[0][i] = *reinterpret_cast<const u32x4*>(pa + (trow + i) * ldx);
        pr[1][i] = *reinterpret_cast<const u32x4*>(pb + (trow + i) * ldx);
      }
      return;
    }
    // edge: element-wise with bounds (tokens beyond the split, features beyond n are 0)
#pragma unroll
    for (int band = 0; band < 2; ++band) {
      const int f0 = band == 0 ? f0a : f0b;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = t0 + tg * 8 + i;
        const bool rowok = t < t_end;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int f = f0 + 2 * d;
          const uint32_t lo = (rowok && f < n) ? (uint32_t)X[t * ldx + f] : 0u;
          const uint32_t hi = (rowok && f + 1 < n) ? (uint32_t)X[t * ldx + f + 1] : 0u;
          pr[band][i][d] = lo | (hi << 16);
        }
      }
    }
  };

  // Transposes part q (band q/2, feature pairs 2*(q%2), 2*(q%2)+1) of a
  // prefetched 8 x 8 block and stores it feature-major into LDS buffer buf.
  auto lstore_part = [&](const u32x4 (&pr)[2][8], int buf, int q) {
    const int band = q >> 1;
#pragma unroll
    for (int f2 = 2 * (q & 1); f2 < 2 * (q & 1) + 2; ++f2) {
      u32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t y = pr[band][2 * e][f2];      // token 2e: features 2f2 (lo) and 2f2+1 (hi)
        const uint32_t x = pr[band][2 * e + 1][f2];  // token 2e+1
        lo[e] = (y & 0xFFFFu) | (x << 16);
        hi[e] = (y >> 16) | (x & 0xFFFF0000u);
      }
      *reinterpret_cast<u32x4*>(&lds[buf][band][fc * 8 + 2 * f2][tg * 8]) = lo;
      *reinterpret_cast<u32x4*>(&lds[buf][band][fc * 8 + 2 * f2 + 1][tg * 8]) = hi;
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

  auto load_a = [&](int buf, int kk, int rb) {
    return *reinterpret_cast<const u32x4*>(&lds[buf][0][arow + rb * 32][kk * 16 + koff]);
  };
  auto load_b = [&](int buf, int kk, u32x4 (&fb)[4]) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      fb[cb] = *reinterpret_cast<const u32x4*>(&lds[buf][1][bcol + cb * 32][kk * 16 + koff]);
  };

  // One stage: 64 MFMAs on LDS buffer buf.  Interleaved with them: the
  // fragment reads that come next (B fragments one 16-token step ahead, A
  // fragments one row block ahead), the transposed LDS stores of the next
  // stage (from prefetch slot nxt, when has_next) and the global loads of the
  // stage after that (into slot fill, when has_fill).  The scheduling hints
  // keep one or two other instructions between MFMAs so that the MFMA pipe
  // does not wait for them.
  auto stage = [&](int buf, u32x4 (&nxt)[2][8], bool has_next, u32x4 (&fill)[2][8], bool has_fill,
                   int64_t fill_t0) {
    if (has_fill) gload(fill, fill_t0);
    u32x4 fb[2][4];
    u32x4 fa[2];
    load_b(buf, 0, fb[0]);
    fa[0] = load_a(buf, 0, 0);
#pragma unroll
    for (int kk = 0; kk < kKt16 / 16; ++kk) {
      if (kk + 1 < kKt16 / 16) load_b(buf, kk + 1, fb[(kk + 1) & 1]);
      if (has_next) lstore_part(nxt, buf ^ 1, kk);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int idx = kk * 4 + rb;
        if (rb + 1 < 4)
          fa[(idx + 1) & 1] = load_a(buf, kk, rb + 1);
        else if (kk + 1 < kKt16 / 16)
          fa[(idx + 1) & 1] = load_a(buf, kk + 1, 0);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[rb][cb] = Mfma16<DT>::run(fa[idx & 1], fb[kk & 1][cb], acc[rb][cb]);
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // up to 2 VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // up to 1 DS read
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // up to 1 DS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // up to 1 VMEM read
      }
    }
  };

  // The next stage is prefetched into registers (slot 0) while this one is
  // multiplied, then transposed into the other LDS buffer.
  gload(pre[0], t_begin);
#pragma unroll
  for (int q = 0; q < 4; ++q) lstore_part(pre[0], 0, q);
  __syncthreads();
  for (int64_t s = 0; s < nstages; ++s) {
    const int buf = (int)(s & 1);
    stage(buf, pre[1], false, pre[0], s + 1 < nstages, t_begin + (s + 1) * kKt16);
    if (s + 1 < nstages) {
#pragma unroll
      for (int q = 0; q < 4; ++q) lstore_part(pre[0], buf ^ 1, q);
    }
    __syncthreads();
  }
  store_acc(acc, dst, wave, lane);
}

// Direct-to-LDS variant for 16-bit X with 8-aligned features (n % 8 == 0,
// ldx % 8 == 0, 16-byte aligned X).  Token rows are copied HBM -> LDS by
// global_load_lds (16 bytes per lane, no register staging): one instruction
// moves one token row of both bands, lanes 0-31 the 256 features of band I
// and lanes 32-63 those of band J, so an LDS row is [band I | band J] (1024
// bytes, padded to 1088 so that the transposing reads below are free of bank
// conflicts).  Lanes whose 8 features lie beyond n copy features 0-7 instead:
// those LDS columns only feed outputs beyond n, which the reduction drops.
// MFMA operands are read with ds_read_b64_tr_b16: within each group of 16
// lanes, lane j receives element j%4 of the 8-byte chunks addressed by lanes
// j/4 + 4e (e = 0..3); with lane j addressing token row t0 + j/4 and
// features f + 4*(j%4), it receives tokens t0..t0+3 of feature f + j, i.e. a
// K-contiguous operand.
//
// Pipeline: stages of 64 tokens (four 16-token MFMA steps) alternate between
// two LDS buffers.  While stage s is multiplied, the loads of stage s+1 go into
// the other buffer (last read before the previous barrier), one per two MFMAs
// of the first two steps, so a wave never waits long at a load for the memory
// pipeline to accept it and the loads have two steps and more to land.  The
// one barrier per stage sits inside the last step, after its first eight
// MFMAs: every wave then holds that step's fragments (buffer s may be refilled
// from the next stage on) and has waited for its own loads of stage s+1
// (visible to all after the barrier); the fragment reads of stage s+1's first
// step overlap the last eight MFMAs.  The last stage of a split may be
// partial: its rows past the split load the split's last row and are zeroed
// once they have landed, before the barrier that publishes the stage.
constexpr int kRowBytes = 1088;
constexpr int kKtD = 64;                        // tokens per stage
constexpr int kSteps = kKtD / 16;               // MFMA steps per stage
constexpr int kNBuf = 2;                        // LDS stage buffers (kNBuf * kStageBytes <= 160 KB)
constexpr int kStageBytes = kKtD * kRowBytes;
constexpr int kRowsPerWave = kKtD / 4;          // direct loads per wave per stage
constexpr int kLoadSteps = 2;                   // steps that issue them, kRowsPerWave / 8 each
constexpr int kDirectLdsBytes = kNBuf * kStageBytes;

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding): vmcnt <= v, expcnt = 7 (no wait), lgkmcnt = 0.
constexpr int waitcnt_vm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4); }

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// orders global memory, which makes every wave drain all of its loads in
// flight at each barrier; the direct-to-LDS loads are waited for explicitly.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int DT>
__global__ __launch_bounds__(kThreads, 1) void syrk16_direct_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int n, int64_t tokens, int nb, int ntiles,
    int nsplit, int64_t tok_per_split, float* __restrict__ partial, int64_t launched) {
  static_assert(kNBuf == 2 && kSteps % 2 == 0 && kLoadSteps < kSteps && kRowsPerWave == 8 * kLoadSteps,
                "pipeline written for two buffers, an even number of steps and 8 loads per loading step");
  // XCD x owns tiles [x*tpx, (x+1)*tpx) of every split (consecutive in the
  // band-blocked order, so they share few bands in its L2) and all XCDs walk
  // the splits in step, so the rows one XCD misses in L2 are the rows the
  // others read at the same time.
  (void)launched;
  const int xcd = (int)(blockIdx.x % kXcds);
  const int64_t idx = blockIdx.x / kXcds;
  const int tpx = (ntiles + kXcds - 1) / kXcds;
  const int t0x = xcd * tpx;
  const int tx = min(ntiles, t0x + tpx) - t0x;
  if (tx <= 0) return;
  const int split = (int)(idx / tx);
  const int tile = t0x + (int)(idx % tx);
  if (split >= nsplit) return;
  int I, J;
  tile_coords(tile, nb, I, J);
  const int64_t t_begin = (int64_t)split * tok_per_split;
  const int64_t t_end = min(tokens, t_begin + tok_per_split);

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  // This lane's 16-byte chunk in a token row: band I for lanes 0-31, band J for 32-63.
  const int band = lane >> 5;
  const int fchunk = (band == 0 ? I : J) * kTile + (lane & 31) * 8;
  const uint32_t lane_bytes = (uint32_t)(fchunk < n ? fchunk : 0) * 2u;  // n % 8 == 0: a chunk is all in or all out

  // Wave w copies token rows 16w .. 16w+15 of a stage.  The row address and
  // the LDS destination are the same for the whole wave (scalar registers);
  // only the 16-byte chunk differs per lane.  Rows past the split are clamped
  // to its last row (a valid address); zero_tail then zeroes them once the
  // wave's own loads have landed.
  //
  // The load is issued by hand: when the compiler sees a direct-to-LDS load
  // it cannot tell which stage buffer it writes, so it would make every
  // later LDS read and the barrier wait for all loads in flight, including
  // the ones just issued for the next stage.  The waits the pipeline needs
  // are explicit (before each barrier).  M0 holds the LDS
  // destination; one wait state separates its write from the load.  The
  // compiler does not keep M0 live across the statement, so the kernel
  // must not index registers dynamically (which would use M0): every
  // fragment and accumulator index here is a compile-time constant.
  auto load_row = [&](int buf, int64_t t0, int i) {
    const int r = wave * kRowsPerWave + i;
    const int64_t t = min(t0 + r, t_end - 1);
    const uint16_t* row = X + t * ldx;
    const uint32_t dst_lds = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)(smem + buf * kStageBytes + r * kRowBytes));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(dst_lds), "v"(lane_bytes), "s"(row) : "memory", "m0");
  };
  auto zero_tail = [&](int buf, int64_t t0) {
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = wave * kRowsPerWave + i;
      if (t0 + r >= t_end)
        *reinterpret_cast<u32x4*>(smem + buf * kStageBytes + r * kRowBytes + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = floatx16{};

  // Transposed-read addressing (see above): group g = lane/16, j = lane%16.
  const int g = lane >> 4, j = lane & 15;
  const int trow = 8 * (g >> 1) + (j >> 2);                 // token row within a 16-token step
  const int fcol = 16 * (g & 1) + 4 * (j & 3);              // feature offset within a 32-feature block
  const int a_off = trow * kRowBytes + (wr * 128 + fcol) * 2;
  const int b_off = trow * kRowBytes + (kTile + wc * 128 + fcol) * 2;

  auto frag = [&](int buf, int off, int kk, int blk) -> u32x4 {
    const unsigned char* p = smem + buf * kStageBytes + off + kk * 16 * kRowBytes + blk * 64;
    const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
    const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p + 4 * kRowBytes));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };

  float* dst = partial + ((int64_t)split * ntiles + tile) * (int64_t)kTileElems;
  const int64_t nstages = (t_end - t_begin + kKtD - 1) / kKtD;
  // Stage st is full when all its rows lie in the split; only the last stage
  // of a split can be partial.
  auto full = [&](int64_t st) { return t_begin + (st + 1) * kKtD <= t_end; };

  u32x4 fa[2][4], fb[2][4];
  // Prologue: stage 0.
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) load_row(0, t_begin, i);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  if (!full(0)) zero_tail(0, t_begin);
  lds_barrier();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) fa[0][rb] = frag(0, a_off, 0, rb);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) fb[0][cb] = frag(0, b_off, 0, cb);
  for (int64_t s = 0; s < nstages; ++s) {
    const int buf = (int)(s & 1);
    const int64_t nt0 = t_begin + (s + 1) * kKtD;          // stage s+1, loaded into buffer buf^1
    const bool more = s + 1 < nstages;
    // Steps 0 .. kSteps-2: the next step's fragments into the other slot and,
    // in the first kLoadSteps steps, eight loads of stage s+1 each.  The last
    // stage loads too (its clamped last row, into the buffer no step reads
    // any more), which keeps the loop free of branches around the loads.
#pragma unroll
    for (int q = 0; q < kSteps - 1; ++q) {
      const int cur = q & 1, nxt = cur ^ 1;
      const bool ld = q < kLoadSteps;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        fa[nxt][k] = frag(buf, a_off, q + 1, k);
        if (ld) load_row(buf ^ 1, nt0, 8 * q + k);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        fb[nxt][k] = frag(buf, b_off, q + 1, k);
        if (ld) load_row(buf ^ 1, nt0, 8 * q + 4 + k);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = Mfma16<DT>::run(fa[cur][rb], fb[cur][cb], acc[rb][cb]);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // a direct-to-LDS load, if any
      }
    }
    // Last step (slot 1): first half of its MFMAs.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = Mfma16<DT>::run(fa[1][rb], fb[1][cb], acc[rb][cb]);
    if (more) {
      // This wave's loads of stage s+1 have landed and its LDS reads of
      // buffer buf are done (lgkmcnt 0) before the barrier publishes the one
      // and frees the other.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      if (!full(s + 1)) zero_tail(buf ^ 1, nt0);
      lds_barrier();
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) fa[0][rb] = frag(buf ^ 1, a_off, 0, rb);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) fb[0][cb] = frag(buf ^ 1, b_off, 0, cb);
    }
#pragma unroll
    for (int rb = 2; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = Mfma16<DT>::run(fa[1][rb], fb[1][cb], acc[rb][cb]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // two LDS reads
    }
  }
  // No load into LDS may still be in flight when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
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
// skip_last drops that many tiles from the end of the band-blocked order.
SyrkPlan plan_syrk(int64_t n, int64_t tokens, int dtype, int skip_last = 0, int max_splits = 1 << 30) {
  SyrkPlan p;
  p.nb = (int)ceil_div(n, kTile);
  p.ntiles = p.nb * (p.nb + 1) / 2 - skip_last;
  const int64_t kt = dtype == GPTQ_F32 ? kKt32 : kKt16;
  const int64_t cus = 256;
  double best = 1e300;
  struct Cand { int s; int64_t tps; double cost; };
  Cand cands[65];
  int nc = 0;
  const int s_min = (int)ceil_div(tokens, kMaxSplitTokens);
  for (int s = s_min; s <= s_min + 64; ++s) {
    if (s > s_min && s > max_splits) break;
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
  // Covers both work mappings: XCD-contiguous items, and per-XCD tile subsets
  // (kXcds x ceil(ntiles / kXcds) tiles per split).
  p.launched = (int64_t)kXcds * ceil_div(p.ntiles, kXcds) * p.nsplit;
  return p;
}

// The plan of a call that leaves out the last skip_last tiles: the token
// splits are those of the full tile set, so the workspace it needs never
// exceeds gptq_hessian_ws_bytes of the full width.
SyrkPlan plan_syrk_skipping(int64_t n, int64_t tokens, int dtype, int skip_last) {
  SyrkPlan p = plan_syrk(n, tokens, dtype);
  if (skip_last > 0) {
    p.ntiles -= skip_last;
    p.launched = (int64_t)kXcds * ceil_div(p.ntiles, kXcds) * p.nsplit;
  }
  return p;
}

size_t plan_ws_bytes(const SyrkPlan& p) {
  return (size_t)p.nsplit * (size_t)p.ntiles * (size_t)kTileElems * sizeof(float);
}

// Tiles of the X_f^T X_f block that a paired call leaves out (0 when they do
// not form the tail of the band-blocked order): with n a multiple of the tile
// and the half a whole number of kGroup-band super-blocks, the tiles with
// both bands in the second half come last.
int pair_skipped_tiles(int64_t n) {
  const int64_t half_bands = ceil_div(n, kTile);
  const bool aligned = n % kTile == 0 && half_bands % kGroup == 0;
  return aligned ? (int)(half_bands * (half_bands + 1) / 2) : 0;
}

// hipFuncSetAttribute once per device and kernel; concurrent first calls may
// both set it (the call is idempotent), none skips it.
std::atomic<uint64_t> g_direct_attr_done[2];

gptq_status ensure_direct_lds_attr(int x_dtype) {
  int dev = 0;
  GPTQ_TRY_HIP(hipGetDevice(&dev));
  const int which = x_dtype == GPTQ_BF16 ? 0 : 1;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit != 0 && (g_direct_attr_done[which].load(std::memory_order_acquire) & bit)) return GPTQ_OK;
  const void* fn = x_dtype == GPTQ_BF16 ? reinterpret_cast<const void*>(&syrk16_direct_kernel<GPTQ_BF16>)
                                        : reinterpret_cast<const void*>(&syrk16_direct_kernel<GPTQ_F16>);
  GPTQ_TRY_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kDirectLdsBytes));
  g_direct_attr_done[which].fetch_or(bit, std::memory_order_release);
  return GPTQ_OK;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_hessian_ws_bytes(int64_t n, int64_t tokens, int x_dtype) {
  if (n <= 0 || tokens <= 0 || !valid_dtype(x_dtype)) return 0;
  return plan_ws_bytes(plan_syrk(n, tokens, x_dtype));
}

extern "C" size_t gptq_hessian_pair_ws_bytes(int64_t n, int64_t tokens, int x_dtype) {
  if (n <= 0 || n > ((int64_t)1 << 15) || tokens <= 0 || !valid_dtype(x_dtype)) return 0;
  return plan_ws_bytes(plan_syrk_skipping(2 * n, tokens, x_dtype, pair_skipped_tiles(n)));
}

namespace {

gptq_status hessian_impl(float* H, int64_t n, const void* X, int x_dtype, int64_t tokens, int64_t ldx, float alpha,
                         int reset, void* ws, size_t ws_bytes, void* stream, int skip_last,
                         int max_splits = 1 << 30) {
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
  const SyrkPlan p = skip_last > 0 ? plan_syrk_skipping(n, tokens, x_dtype, skip_last)
                                   : plan_syrk(n, tokens, x_dtype, 0, max_splits);
  const size_t need = plan_ws_bytes(p);
  if (ws == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  float* partial = static_cast<float*>(ws);
  if (x_dtype == GPTQ_F32) {
    syrk32_kernel<<<(unsigned)p.launched, kThreads, 0, st>>>(
        static_cast<const float*>(X), ldx, (int)n, tokens, p.nb, p.ntiles, p.nsplit, p.tok_per_split,
        partial, p.launched);
  } else {
    const int vec_ok = (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    const bool direct = vec_ok && (n % 8 == 0);
    if (direct) {
      const gptq_status rc = ensure_direct_lds_attr(x_dtype);
      if (rc != GPTQ_OK) return rc;
      if (x_dtype == GPTQ_BF16)
        syrk16_direct_kernel<GPTQ_BF16><<<(unsigned)p.launched, kThreads, kDirectLdsBytes, st>>>(
            static_cast<const uint16_t*>(X), ldx, (int)n, tokens, p.nb, p.ntiles, p.nsplit, p.tok_per_split,
            partial, p.launched);
      else
        syrk16_direct_kernel<GPTQ_F16><<<(unsigned)p.launched, kThreads, kDirectLdsBytes, st>>>(
            static_cast<const uint16_t*>(X), ldx, (int)n, tokens, p.nb, p.ntiles, p.nsplit, p.tok_per_split,
            partial, p.launched);
    } else if (x_dtype == GPTQ_BF16)
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

}  // namespace

namespace gptq {

int64_t hessian_split_bytes(int64_t n) {
  const int64_t nb = ceil_div(n, kTile);
  return nb * (nb + 1) / 2 * (int64_t)kTileElems * (int64_t)sizeof(float);
}

gptq_status hessian_accumulate_bounded(float* H, int64_t n, const void* X, int x_dtype, int64_t tokens,
                                       int64_t ldx, float alpha, int reset, void* ws, size_t ws_bytes,
                                       void* stream) {
  if (n < 0 || tokens < 0 || !valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (n > (int64_t)1 << 16) return GPTQ_ERR_UNSUPPORTED;
  if (n == 0) return GPTQ_OK;
  if (H == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (tokens > 0 && (X == nullptr || ldx < n)) return GPTQ_ERR_INVALID_ARG;
  const int64_t per_split = hessian_split_bytes(n);
  const int64_t max_splits = (int64_t)ws_bytes / per_split;
  if (ws == nullptr || max_splits < 1) return GPTQ_ERR_WORKSPACE;
  if (tokens == 0) return hessian_impl(H, n, X, x_dtype, 0, ldx, alpha, reset, ws, ws_bytes, stream, 0);
  // Passes of at most max_splits splits of kMaxSplitTokens tokens; each pass
  // adds its float64 split sum to H (the first pass honours reset).
  const int64_t pass_tokens = max_splits * kMaxSplitTokens;
  const char* xb = static_cast<const char*>(X);
  for (int64_t t0 = 0; t0 < tokens; t0 += pass_tokens) {
    const int64_t tt = std::min(pass_tokens, tokens - t0);
    const gptq_status rc = hessian_impl(H, n, xb + t0 * ldx * (int64_t)elem_bytes(x_dtype), x_dtype, tt, ldx,
                                        alpha, t0 == 0 ? reset : 0, ws, ws_bytes, stream, 0, (int)max_splits);
    if (rc != GPTQ_OK) return rc;
  }
  return GPTQ_OK;
}

}  // namespace gptq

extern "C" gptq_status gptq_hessian_accumulate(float* H, int64_t n, const void* X, int x_dtype,
                                               int64_t tokens, int64_t ldx, float alpha, int reset,
                                               void* ws, size_t ws_bytes, void* stream) {
  return hessian_impl(H, n, X, x_dtype, tokens, ldx, alpha, reset, ws, ws_bytes, stream, 0);
}

extern "C" gptq_status gptq_hessian_pair_accumulate(float* H2, int64_t n, const void* Xcat, int x_dtype,
                                                    int64_t tokens, int64_t ldx, float alpha, int reset,
                                                    void* ws, size_t ws_bytes, void* stream) {
  if (n < 0) return GPTQ_ERR_INVALID_ARG;
  if (n > ((int64_t)1 << 15)) return GPTQ_ERR_UNSUPPORTED;
  return hessian_impl(H2, 2 * n, Xcat, x_dtype, tokens, ldx, alpha, reset, ws, ws_bytes, stream,
                      pair_skipped_tiles(n));
}
