// Library-internal entry of the Hessian accumulation for callers that bring
// a workspace of a fixed size (the allocation-free entry point).
#pragma once

#include "common.h"

namespace gptq {

// Bytes of the partial upper tiles of one token split at width n.
int64_t hessian_split_bytes(int64_t n);

// gptq_hessian_accumulate with whatever workspace is given: the tokens are
// taken in passes of as many token splits as ws holds, each pass adding its
// float64 split sum into H.  Needs ws_bytes >= hessian_split_bytes(n).
gptq_status hessian_accumulate_bounded(float* H, int64_t n, const void* X, int x_dtype, int64_t tokens,
                                       int64_t ldx, float alpha, int reset, void* ws, size_t ws_bytes,
                                       void* stream);

}  // namespace gptq
