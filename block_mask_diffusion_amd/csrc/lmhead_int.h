// Internal interface between the LM-head sources (not part of the C ABI).
#pragma once

#include "common.h"

// k-stage width of the large-M kernel; H must be a multiple of it for that kernel to apply.
#ifndef TT_GEMM_KB
#define TT_GEMM_KB 64
#endif

// Launches the MFMA GEMM LM-head kernel (bf16, H % TT_GEMM_KB == 0; used for M > 16) on stream s.
__attribute__((visibility("hidden"))) int tt_lm_gemm_launch(const void* hidden, const void* w,
                                                            float* logits, int M, int H, int V,
                                                            hipStream_t s);

// Vocabulary columns of one wave's block in the GEMM kernel's tile for (M, V): 64 or 128.
__attribute__((visibility("hidden"))) int tt_lm_gemm_cols(int M, int V);

struct TtRedArgs;
// Fused variant of the GEMM kernel: instead of logits, one (max, lowest argmax, sum exp) record
// per (row, column block of one wave) in red.parts (red.nparts = ceil(V / tt_lm_gemm_cols(M, V))).
__attribute__((visibility("hidden"))) int tt_lm_gemm_reduce_launch(const void* hidden, const void* w,
                                                                   int M, int H, int V, TtRedArgs red,
                                                                   hipStream_t s);

// Fused LM head + vocabulary reduction (bf16, H % TT_GEMM_KB == 0): records per row, and launch.
__attribute__((visibility("hidden"))) int tt_lm_reduce_nparts(int M, int H, int V);
__attribute__((visibility("hidden"))) int tt_lm_reduce_launch(const void* hidden, const void* w, int M, int H,
                                                              int V, TtRedArgs red, hipStream_t s);
