// Host-CPU MXFP4 SwiGLU expert kernel (reads blobs in the pool's layout).
#pragma once
#include "moe_internal.h"

namespace moe {

// "avx512" or "scalar": the instruction set the kernel runs with on this host
// (MOE_HOST_FFN_SCALAR=1 in the environment forces the scalar code)
const char* host_ffn_isa();

// y[H] (FP32) = sum_j w[j] * FFN_j(x) over n experts (blobs in the pool's
// layout, host memory), x[H] bf16; experts are shared out over `threads`
// threads and their partial sums added in thread order.
void host_expert_ffn(const Layout& L, const uint8_t* const* blobs, const float* w, int n, const uint16_t* x,
                     float* y, int threads);

// bytes of blob processed per second by `threads` threads running the kernel
// over blobs[0..n) round robin for about min_seconds
double host_expert_rate(const Layout& L, const uint8_t* const* blobs, int n, int threads, double min_seconds);

}  // namespace moe
