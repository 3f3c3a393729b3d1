// Confidence unmasking ("Nemotron-Labs-TwoTower" wiki page, section "Block-wise generation").
//
// Two kernels on the caller's stream:
//   unmask_partial  one workgroup per (still-masked row, 4096-entry vocabulary chunk): streams the
//                   chunk once with coalesced 16-byte loads and reduces it to (max, lowest argmax,
//                   sum of exp(l - max)), the mask id's logit counting as -inf. HBM-bound: each
//                   logit of a masked row is read exactly once; rows already committed are skipped
//                   without reading anything but their mask word.
//   unmask_commit   one workgroup per block: row i's chunk partials are merged in a fixed order
//                   (deterministic) by four waves in parallel; lane i of wave 0 then holds
//                   conf = 1 / sum and the prediction and applies the threshold, the completion
//                   floor and the in-place token / bitmap update.
//
// The fused LM head + unmask call (tt_lmhead_unmask) replaces the logits and unmask_partial with
// the LM-head kernels' reduction epilogue (one record per row and column block of one wave),
// merges each masked row's records with unmask_rowmerge and ends with the same unmask_commit.
#include <mutex>

#include "lmhead_int.h"
#include "reduce_int.h"

namespace {

constexpr int UM_THREADS = 256;
#ifndef TT_UM_PER_THREAD
#define TT_UM_PER_THREAD 16
#endif
constexpr int UM_PER_THREAD = TT_UM_PER_THREAD;
constexpr int UM_CHUNK = UM_THREADS * UM_PER_THREAD;  // vocabulary entries per workgroup
typedef TtPartial Partial;

// c = log2(e) / temperature: every record's sum is sum exp2((l - m) c)
__device__ __forceinline__ void merge(float& m, int& a, float& s, float m2, int a2, float s2, float c) {
  tt_merge(m, a, s, m2, a2, s2, c);
}

// Merges the records of the workgroup's UM_THREADS threads in a fixed order (butterfly inside each
// wave, then the waves in increasing order) and stores the result to *out from thread 0.
__device__ __forceinline__ void wg_merge_store(float m, int a, float s, Partial* out, float c) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = tt_shfl_xor(m, off);
    int a2 = tt_shfl_xor(a, off);
    float s2 = tt_shfl_xor(s, off);
    merge(m, a, s, m2, a2, s2, c);
  }
  __shared__ float sm[UM_THREADS / TT_WAVE], ss[UM_THREADS / TT_WAVE];
  __shared__ int sa[UM_THREADS / TT_WAVE];
  const int t = threadIdx.x, w = t / TT_WAVE;
  if ((t & (TT_WAVE - 1)) == 0) {
    sm[w] = m;
    ss[w] = s;
    sa[w] = a;
  }
  __syncthreads();
  if (t == 0) {
    for (int k = 1; k < UM_THREADS / TT_WAVE; ++k) merge(m, a, s, sm[k], sa[k], ss[k], c);
    Partial p;
    p.m = m;
    p.s = s;
    p.a = a;
    p.pad = 0;
    *out = p;
  }
}

template <bool VEC4>
__global__ __launch_bounds__(UM_THREADS) void unmask_partial(const float* __restrict__ logits,
                                                             const uint64_t* __restrict__ mask_bits,
                                                             Partial* __restrict__ ws, int S, int V,
                                                             int nchunk, int mask_id, float cs) {
  const int r = blockIdx.x / nchunk;
  const int c = blockIdx.x - r * nchunk;
  const int b = r / S, i = r - b * S;
  if (!((mask_bits[b] >> i) & 1ull)) return;  // committed rows are never read
  const float* row = logits + (size_t)r * V;
  const int t = threadIdx.x;
  const int v0 = c * UM_CHUNK;

  float x[UM_PER_THREAD];
  int idx[UM_PER_THREAD];
  if (VEC4) {
    // slot k: index v0 + (k/4)*1024 + 4t + k%4 -> each load instruction covers 4 KiB contiguous
#pragma unroll
    for (int q = 0; q < UM_PER_THREAD / 4; ++q) {
      int base = v0 + q * (UM_THREADS * 4) + 4 * t;
      f32x4 val;
      if (base + 3 < V) {
        val = *reinterpret_cast<const f32x4*>(row + base);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (base + e < V) ? row[base + e] : -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[4 * q + e] = val[e];
        idx[4 * q + e] = base + e;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < UM_PER_THREAD; ++k) {
      int v = v0 + k * UM_THREADS + t;
      x[k] = (v < V) ? row[v] : -INFINITY;
      idx[k] = v;
    }
  }
  // the mask token never competes; indices grow with k, so a strict '>' keeps the lowest index
  float m = -INFINITY;
  int a = INT32_MAX;
#pragma unroll
  for (int k = 0; k < UM_PER_THREAD; ++k) {
    if (idx[k] == mask_id) x[k] = -INFINITY;
    if (x[k] > m) {
      m = x[k];
      a = idx[k];
    }
  }
  float s = 0.f;
  if (m != -INFINITY) {
    const float mb = m * cs;
#pragma unroll
    for (int k = 0; k < UM_PER_THREAD; ++k) s += tt_exp2(fmaf(x[k], cs, -mb));
  }
  wg_merge_store(m, a, s, ws + (size_t)r * nchunk + c, cs);
}

// One workgroup per (block, position) of the fused path: the row's nparts records (one per column
// block of one LM-head wave) are merged, thread t taking records t, t + 256, ... in increasing
// order, then across the workgroup in a fixed order; committed positions are skipped.
constexpr int RM_BATCH = 4;
__global__ __launch_bounds__(UM_THREADS) void unmask_rowmerge(const Partial* __restrict__ parts,
                                                              const uint64_t* __restrict__ mask_bits,
                                                              Partial* __restrict__ rowres, int S,
                                                              int nparts, float cs) {
  const int r = blockIdx.x;
  const int b = r / S, i = r - b * S;
  if (!((mask_bits[b] >> i) & 1ull)) return;
  const Partial* p = parts + (size_t)r * nparts;
  float m = -INFINITY, s = 0.f;
  int a = INT32_MAX;
  for (int c0 = threadIdx.x; c0 < nparts; c0 += UM_THREADS * RM_BATCH) {
    Partial x[RM_BATCH];
#pragma unroll
    for (int k = 0; k < RM_BATCH; ++k) {
      const int c = c0 + UM_THREADS * k;
      if (c < nparts) x[k] = p[c];
      else x[k] = Partial{-INFINITY, 0.f, INT32_MAX, 0};
    }
#pragma unroll
    for (int k = 0; k < RM_BATCH; ++k) merge(m, a, s, x[k].m, x[k].a, x[k].s, cs);
  }
  wg_merge_store(m, a, s, rowres + r, cs);
}

constexpr int CM_THREADS = 256;
constexpr int CM_Q = CM_THREADS / TT_WAVE;  // chunk stripes merged in parallel per row
constexpr int CM_BATCH = 8;                 // partial loads issued before merging

// One workgroup per block. Thread (stripe q, row i) merges the partials c = q, q+4, q+8, ... of
// row i, issuing a batch of loads before merging them in increasing c; wave 0 then merges the four
// stripes in the order q = 0..3 (a fixed order: bitwise reproducible), so lane i holds row i's
// confidence and prediction, and applies the commit rule for the block:
//   kind TT_SAMPLER_CONFIDENCE: conf >= gamma, topped up to the completion floor;
//   kind TT_SAMPLER_PREDICT_NOISE: the n_masked - floor(S (T-1-step) / T) most confident.
__global__ __launch_bounds__(CM_THREADS) void unmask_commit(const Partial* __restrict__ ws,
                                                           int32_t* __restrict__ tokens,
                                                           uint64_t* __restrict__ mask_bits,
                                                           int32_t* __restrict__ n_masked,
                                                           float* __restrict__ conf_out,
                                                           int32_t* __restrict__ pred_out, int S,
                                                           int nchunk, int step, int num_steps,
                                                           int kind, float gamma, float cs) {
  __shared__ float pm[CM_Q][TT_WAVE], ps[CM_Q][TT_WAVE];
  __shared__ int pa[CM_Q][TT_WAVE];
  const int b = blockIdx.x;
  const int i = threadIdx.x & (TT_WAVE - 1), q = threadIdx.x / TT_WAVE;
  const uint64_t bits = mask_bits[b];
  const bool masked = (i < S) && ((bits >> i) & 1ull);
  float m = -INFINITY, s = 0.f;
  int a = INT32_MAX;
  // Every row of the block loads its records without waiting for the mask word (a row that is not
  // masked holds stale records, in bounds, that are dropped below): one memory round trip less.
  if (i < S) {
    const Partial* p = ws + (size_t)(b * S + i) * nchunk;
    for (int c0 = q; c0 < nchunk; c0 += CM_Q * CM_BATCH) {
      Partial x[CM_BATCH];
#pragma unroll
      for (int k = 0; k < CM_BATCH; ++k) {
        const int c = c0 + CM_Q * k;
        if (c < nchunk) x[k] = p[c];
        else x[k] = Partial{-INFINITY, 0.f, INT32_MAX, 0};
      }
#pragma unroll
      for (int k = 0; k < CM_BATCH; ++k) merge(m, a, s, x[k].m, x[k].a, x[k].s, cs);
    }
  }
  if (!masked) {
    m = -INFINITY;
    s = 0.f;
    a = INT32_MAX;
  }
  pm[q][i] = m;
  ps[q][i] = s;
  pa[q][i] = a;
  __syncthreads();
  if (q != 0) return;
#pragma unroll
  for (int k = 1; k < CM_Q; ++k) merge(m, a, s, pm[k][i], pa[k][i], ps[k][i], cs);
  float conf = -1.f;
  int pred = -1;
  if (masked) {
    conf = 1.f / s;
    pred = a;
  }
  const uint64_t mk = __ballot(masked);
  const int nM = __popcll(mk);
  uint64_t sel = 0;
  if (nM > 0) {
    int k;
    if (kind == TT_SAMPLER_PREDICT_NOISE) {
      const int target = (S * (num_steps - 1 - step)) / num_steps;  // linear schedule
      k = max(nM - target, 0);
      sel = 0;
    } else {
      sel = __ballot(masked && conf >= gamma);
      const int left = num_steps - step;
      k = (nM + left - 1) / left;  // completion floor
    }
    if (__popcll(sel) < k) {
      int rank = 0;  // place among the masked positions: higher conf first, then lower position
      for (int j = 0; j < S; ++j) {  // j is uniform: a scalar read of lane j
        const float cj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(conf), j));
        bool mj = (mk >> j) & 1ull;
        rank += (mj && (cj > conf || (cj == conf && j < i))) ? 1 : 0;
      }
      sel = __ballot(masked && rank < k);
    }
  }
  if ((sel >> i) & 1ull) tokens[(size_t)b * S + i] = pred;
  if (i < S) {
    if (conf_out) conf_out[(size_t)b * S + i] = conf;
    if (pred_out) pred_out[(size_t)b * S + i] = pred;
  }
  if (i == 0) {
    mask_bits[b] = bits & ~sel;
    n_masked[b] = nM - __popcll(sel);
  }
}

// Host checks shared by the unmask entry points.
int unmask_check(const int32_t* tokens, const uint64_t* mask_bits, const int32_t* n_masked,
                 const size_t* workspace_bytes, int B, int S, int V, int step, int num_steps,
                 int mask_id, const tt_sampler* sm) {
  if (!tokens || !mask_bits || !n_masked || !workspace_bytes || !sm) return TT_ERR_ARG;
  if (B <= 0 || S <= 0 || V < 2) return TT_ERR_ARG;
  if (mask_id < 0 || mask_id >= V) return TT_ERR_ARG;
  if (num_steps <= 0 || step < 0 || step >= num_steps) return TT_ERR_ARG;
  if (sm->gamma != sm->gamma) return TT_ERR_ARG;
  if (!(sm->temperature > 0.f) || !isfinite(sm->temperature)) return TT_ERR_ARG;
  if (sm->kind != TT_SAMPLER_CONFIDENCE && sm->kind != TT_SAMPLER_PREDICT_NOISE) return TT_ERR_UNSUPPORTED;
  return TT_OK;
}

float sampler_scale(const tt_sampler* sm) { return TT_LOG2E / sm->temperature; }

// Records of the unmasking step's first kernel: one per (row, vocabulary chunk).
size_t unmask_records(int B, int S, int V) {
  return (size_t)B * S * (size_t)((V + UM_CHUNK - 1) / UM_CHUNK);
}

// The two kernels of an unmasking step, with `ws` holding unmask_records(B, S, V) records
// (arguments already checked).
int unmask_launch(const float* logits, int32_t* tokens, uint64_t* mask_bits, int32_t* n_masked,
                  float* conf_out, int32_t* pred_out, int B, int S, int V, int step, int num_steps,
                  const tt_sampler* sampler, int mask_id, Partial* ws, hipStream_t s) {
  const size_t rows = (size_t)B * S;
  const int nchunk = (V + UM_CHUNK - 1) / UM_CHUNK;
  const float cs = sampler_scale(sampler);
  const bool vec4 = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0);
  dim3 grid((unsigned)(rows * nchunk));
  if (vec4)
    hipLaunchKernelGGL(unmask_partial<true>, grid, dim3(UM_THREADS), 0, s, logits, mask_bits, ws,
                       S, V, nchunk, mask_id, cs);
  else
    hipLaunchKernelGGL(unmask_partial<false>, grid, dim3(UM_THREADS), 0, s, logits, mask_bits, ws,
                       S, V, nchunk, mask_id, cs);
  if (tt_launch_status() != TT_OK) return TT_ERR_HIP;
  hipLaunchKernelGGL(unmask_commit, dim3(B), dim3(CM_THREADS), 0, s, ws, tokens, mask_bits, n_masked,
                     conf_out, pred_out, S, nchunk, step, num_steps, sampler->kind, sampler->gamma, cs);
  return tt_launch_status();
}

// Scratch of tt_confidence_unmask_noalloc: the records of unmask_launch in a fixed array of each
// device (every GPU the library runs on holds it until the process ends). Host code never uses
// the array's name as an address: the device address is looked up once per device.
constexpr size_t UM_SCRATCH_BYTES = (size_t)2 << 20;
static __device__ __align__(256) unsigned char scratch[UM_SCRATCH_BYTES];
constexpr int UM_MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[UM_MAX_DEVICES];

// Device address of `scratch` on the current device (nullptr if the lookup fails).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= UM_MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_dev[dev] = p;
  }
  return scratch_dev[dev];
}

}  // namespace

extern "C" int tt_unmask_sample(const float* logits, int32_t* tokens, uint64_t* mask_bits,
                                int32_t* n_masked, float* conf_out, int32_t* pred_out, int B, int S,
                                int V, int step, int num_steps, const tt_sampler* sampler, int mask_id,
                                void* workspace, size_t* workspace_bytes, void* stream) {
  if (!logits) return TT_ERR_ARG;
  int st = unmask_check(tokens, mask_bits, n_masked, workspace_bytes, B, S, V, step, num_steps, mask_id,
                        sampler);
  if (st != TT_OK) return st;
  if (S > 64) return TT_ERR_UNSUPPORTED;
  const size_t recs = unmask_records(B, S, V);
  if (recs > (size_t)INT32_MAX) return TT_ERR_UNSUPPORTED;
  st = tt_workspace_check(workspace, workspace_bytes, recs * sizeof(Partial));
  if (st != 0) return st < 0 ? st : TT_OK;
  if ((uintptr_t)workspace % alignof(Partial)) return TT_ERR_ARG;
  return unmask_launch(logits, tokens, mask_bits, n_masked, conf_out, pred_out, B, S, V, step, num_steps,
                       sampler, mask_id, (Partial*)workspace, (hipStream_t)stream);
}

extern "C" int tt_confidence_unmask_noalloc(const float* logits, int32_t* tokens, uint64_t* mask_bits,
                                            int32_t* n_masked, float* conf_out, int32_t* pred_out, int B,
                                            int S, int V, int step, int num_steps, float gamma, int mask_id,
                                            void* stream) {
  if (!logits) return TT_ERR_ARG;
  const tt_sampler sm{TT_SAMPLER_CONFIDENCE, gamma, 1.f};
  size_t unused = 0;
  int st = unmask_check(tokens, mask_bits, n_masked, &unused, B, S, V, step, num_steps, mask_id, &sm);
  if (st != TT_OK) return st;
  if (S > 64) return TT_ERR_UNSUPPORTED;
  if (unmask_records(B, S, V) * sizeof(Partial) > UM_SCRATCH_BYTES) return TT_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return TT_ERR_HIP;
  return unmask_launch(logits, tokens, mask_bits, n_masked, conf_out, pred_out, B, S, V, step, num_steps, &sm,
                       mask_id, (Partial*)ws, (hipStream_t)stream);
}

extern "C" int tt_confidence_unmask(const float* logits, int32_t* tokens, uint64_t* mask_bits,
                                    int32_t* n_masked, float* conf_out, int32_t* pred_out, int B,
                                    int S, int V, int step, int num_steps, float gamma,
                                    int mask_id, void* workspace, size_t* workspace_bytes,
                                    void* stream) {
  const tt_sampler sm{TT_SAMPLER_CONFIDENCE, gamma, 1.f};
  return tt_unmask_sample(logits, tokens, mask_bits, n_masked, conf_out, pred_out, B, S, V, step, num_steps,
                          &sm, mask_id, workspace, workspace_bytes, stream);
}

extern "C" int tt_lmhead_unmask(const void* hidden, const void* w, const int32_t* bias_tok,
                                const float* bias_val, int32_t* tokens, uint64_t* mask_bits,
                                int32_t* n_masked, float* conf_out, int32_t* pred_out, int B, int S,
                                int H, int V, int step, int num_steps, const tt_sampler* sampler,
                                int mask_id, int dtype, void* workspace, size_t* workspace_bytes,
                                void* stream) {
  if (!hidden || !w) return TT_ERR_ARG;
  if ((bias_tok == nullptr) != (bias_val == nullptr)) return TT_ERR_ARG;
  int st = unmask_check(tokens, mask_bits, n_masked, workspace_bytes, B, S, V, step, num_steps, mask_id,
                        sampler);
  if (st != TT_OK) return st;
  if (H <= 0) return TT_ERR_ARG;
  if (dtype != TT_F32 && dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (dtype != TT_BF16 || H % TT_GEMM_KB != 0 || S > 64) return TT_ERR_UNSUPPORTED;
  if ((size_t)B * S > (size_t)INT32_MAX) return TT_ERR_UNSUPPORTED;
  const int M = B * S;
  const int nparts = tt_lm_reduce_nparts(M, H, V);
  if ((size_t)M * nparts > (size_t)INT32_MAX) return TT_ERR_UNSUPPORTED;
  const size_t parts_bytes = (size_t)M * nparts * sizeof(Partial);
  const size_t need = parts_bytes + (size_t)M * sizeof(Partial);
  st = tt_workspace_check(workspace, workspace_bytes, need);
  if (st != 0) return st < 0 ? st : TT_OK;
  if ((uintptr_t)workspace % alignof(Partial)) return TT_ERR_ARG;
  if ((uintptr_t)hidden % 16 || (uintptr_t)w % 16) return TT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  Partial* parts = (Partial*)workspace;
  Partial* rowres = (Partial*)((char*)workspace + parts_bytes);
  const float cs = sampler_scale(sampler);
  const TtRedArgs red{bias_tok, bias_val, mask_id, parts, nparts, mask_bits, S, B, cs};
  if (tt_lm_reduce_launch(hidden, w, M, H, V, red, s) != TT_OK) return TT_ERR_HIP;
  hipLaunchKernelGGL(unmask_rowmerge, dim3((unsigned)M), dim3(UM_THREADS), 0, s, parts, mask_bits, rowres,
                     S, nparts, cs);
  if (tt_launch_status() != TT_OK) return TT_ERR_HIP;
  hipLaunchKernelGGL(unmask_commit, dim3(B), dim3(CM_THREADS), 0, s, rowres, tokens, mask_bits, n_masked,
                     conf_out, pred_out, S, 1, step, num_steps, sampler->kind, sampler->gamma, cs);
  return tt_launch_status();
}
