// Stage 4: pack the codes (GPTQ knowledge note, "Tradeoffs": deployment runs
// on packed weights; Wiki "GPTQ", "Performance and Accuracy": 4 bits per
// weight).  Row-wise little-endian bit stream in 32-bit words: the code of
// column k occupies bits [k*b, (k+1)*b).  One thread packs 32 codes into b
// whole words (read as two 16-byte loads, 4- and 2-bit words written as one
// 16- or 8-byte store), so reads and writes of neighbouring threads are
// contiguous.
#include "common.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;

template <int BITS>
__device__ inline void pack32(const uint8_t* src, int count, uint32_t (&out)[BITS]) {
  // 32 codes as bytes: two 16-byte reads when the segment is whole and
  // aligned (rows of a multiple of 16 codes), else one byte at a time.
  uint32_t b[8];
  if (count == 32 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    const uint4 lo = *reinterpret_cast<const uint4*>(src);
    const uint4 hi = *reinterpret_cast<const uint4*>(src + 16);
    b[0] = lo.x; b[1] = lo.y; b[2] = lo.z; b[3] = lo.w;
    b[4] = hi.x; b[5] = hi.y; b[6] = hi.z; b[7] = hi.w;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t v = 0u;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (4 * q + t < count) v |= (uint32_t)src[4 * q + t] << (8 * t);
      b[q] = v;
    }
  }
#pragma unroll
  for (int w = 0; w < BITS; ++w) out[w] = 0u;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint32_t c = (b[k >> 2] >> (8 * (k & 3))) & 0xffu;
    const int bit = k * BITS;
    out[bit >> 5] |= c << (bit & 31);
    if ((bit & 31) + BITS > 32) out[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
  }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint8_t* __restrict__ codes, int n,
                                                        uint32_t* __restrict__ packed, int64_t ldp) {
  const int64_t r = blockIdx.x;
  const uint8_t* src = codes + r * n;
  uint32_t* dst = packed + r * ldp;
  const int nseg = (n + 31) / 32;
  const int nwords = (int)(((int64_t)n * BITS + 31) / 32);
  // Whole segments of an aligned row go out in one store of BITS words (4-
  // and 2-bit codes; 3-bit words go out one by one).
  const bool vec = BITS != 3 && (reinterpret_cast<uintptr_t>(dst) & (4 * BITS - 1)) == 0;
  for (int sg = threadIdx.x; sg < nseg; sg += kThreads) {
    uint32_t out[BITS];
    pack32<BITS>(src + sg * 32, min(32, n - sg * 32), out);
    if (vec && sg * BITS + BITS <= nwords) {
      if constexpr (BITS == 4) {
        *reinterpret_cast<uint4*>(dst + sg * 4) = uint4{out[0], out[1], out[2], out[3]};
      } else if constexpr (BITS == 2) {
        *reinterpret_cast<uint2*>(dst + sg * 2) = uint2{out[0], out[1]};
      }
    } else {
#pragma unroll
      for (int w = 0; w < BITS; ++w) {
        const int wi = sg * BITS + w;
        if (wi < nwords) dst[wi] = out[w];
      }
    }
  }
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" gptq_status gptq_pack(const uint8_t* codes, int64_t m, int64_t n, int bits, uint32_t* packed,
                                 int64_t ld_packed, void* stream) {
  if (m < 0 || n < 0) return GPTQ_ERR_INVALID_ARG;
  if (!(bits == 2 || bits == 3 || bits == 4)) return GPTQ_ERR_INVALID_ARG;
  if (n > (int64_t)1 << 16 || m > ((int64_t)1 << 31) - 1) return GPTQ_ERR_UNSUPPORTED;
  if (n == 0 || m == 0) return GPTQ_OK;
  if (codes == nullptr || packed == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (ld_packed < ceil_div(n * bits, 32)) return GPTQ_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)m;
  if (bits == 2)
    pack_kernel<2><<<grid, kThreads, 0, st>>>(codes, (int)n, packed, ld_packed);
  else if (bits == 3)
    pack_kernel<3><<<grid, kThreads, 0, st>>>(codes, (int)n, packed, ld_packed);
  else
    pack_kernel<4><<<grid, kThreads, 0, st>>>(codes, (int)n, packed, ld_packed);
  GPTQ_TRY_LAUNCH();
  return GPTQ_OK;
}

extern "C" const char* gptq_status_string(int status) {
  switch (status) {
    case GPTQ_OK: return "GPTQ_OK";
    case GPTQ_ERR_INVALID_ARG: return "GPTQ_ERR_INVALID_ARG";
    case GPTQ_ERR_UNSUPPORTED: return "GPTQ_ERR_UNSUPPORTED";
    case GPTQ_ERR_WORKSPACE: return "GPTQ_ERR_WORKSPACE";
    case GPTQ_ERR_NOT_PD: return "GPTQ_ERR_NOT_PD";
    case GPTQ_ERR_HIP: return "GPTQ_ERR_HIP";
    default: return "GPTQ_UNKNOWN_STATUS";
  }
}
