// Internal interface between the LM-head sources (not part of the C ABI).
#pragma once

#include "common.h"

// k-stage width of the large-M kernel; H must be a multiple of it for that kernel to apply.
#define TT_GEMM_KB 64

// Launches the MFMA GEMM LM-head kernel (bf16, H % TT_GEMM_KB == 0; used for M > 64) on stream s.
__attribute__((visibility("hidden"))) int tt_lm_gemm_launch(const void* hidden, const void* w,
                                                            float* logits, int M, int H, int V,
                                                            hipStream_t s);
