// Confidence unmasking ("Nemotron-Labs-TwoTower" wiki page, section "Block-wise generation").
//
// One kernel on the caller's stream, unmask_step. Row r (position i of block b) is split into
// nsplit ranges of 4096-entry vocabulary chunks, one workgroup per (row, range), with nsplit chosen
// so that the grid holds about 1024 workgroups. A workgroup of a still-masked row streams its
// range once with coalesced 16-byte loads and reduces it to a record (max, lowest argmax, sum of
// exp(l - max)), the mask id's logit counting as -inf; rows already committed read nothing but
// their mask word. Two levels of arrival tickets then finish the step inside the same launch: the
// last workgroup of a row to arrive merges the row's records into one, and the last row of a
// block to arrive commits the block: lane i of its first wave holds conf = 1 / sum and the
// prediction of position i and applies the threshold, the completion floor and the in-place
// token / bitmap update. Records are merged in a fixed order whichever workgroup arrives last, so
// results are bitwise reproducible. Every counter is reset to zero by its last arriver.
//
// The fused LM head + unmask call (tt_lmhead_unmask) replaces the logits and the chunk reduction
// with the LM-head kernels' reduction epilogue (one record per row and column block of one wave);
// unmask_rowstep merges each masked row's records (one workgroup per row) and commits the block
// through the block ticket.
#include <algorithm>
#include <mutex>

#include "lmhead_int.h"
#include "reduce_int.h"

namespace {

constexpr int UM_THREADS = 256;
constexpr int UM_PER_THREAD = 16;
constexpr int UM_CHUNK = UM_THREADS * UM_PER_THREAD;  // vocabulary entries per chunk
constexpr int UM_TARGET_WG = 1024;                    // workgroups the row split aims at
// Counter slots are 64 bytes apart, so the tickets of different rows and blocks never contend
// for one cache line.
constexpr int UM_SLOT = 16;
constexpr size_t UM_SLOT_BYTES = UM_SLOT * sizeof(unsigned);
typedef TtPartial Partial;

// Records that one workgroup stores and a later-arriving workgroup (possibly on another XCD,
// behind another L2) reads: both sides use agent-scope relaxed atomics, which the memory system
// keeps coherent across the XCDs' L2 caches without a whole-L2 writeback or invalidate.
__device__ __forceinline__ void store_record(Partial* out, float m, float s, int a) {
  const uint64_t lo = (uint64_t)__float_as_uint(m) | ((uint64_t)__float_as_uint(s) << 32);
  const uint64_t hi = (uint64_t)(uint32_t)a;
  __hip_atomic_store(reinterpret_cast<uint64_t*>(out), lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(out) + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ Partial load_record(const Partial* in) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<Partial*>(in));
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return Partial{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)), (int)(uint32_t)hi, 0};
}

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
    store_record(out, m, s, a);
  }
}

// Chunk [v0, v0 + UM_CHUNK) of one logits row, the calling thread's UM_PER_THREAD entries (those
// past V read as -inf). VEC4: entry k is v0 + (k/4)*1024 + 4t + k%4, so each load instruction
// covers 4 KiB contiguous; otherwise entry k is v0 + 256k + t.
template <bool VEC4>
__device__ __forceinline__ int chunk_index(int v0, int k) {
  const int t = threadIdx.x;
  return VEC4 ? v0 + (k / 4) * (UM_THREADS * 4) + 4 * t + k % 4 : v0 + k * UM_THREADS + t;
}
// A chunk that lies wholly inside the row: loads without bounds checks.
template <bool VEC4>
__device__ __forceinline__ void chunk_load(const float* __restrict__ row, int v0, float (&x)[UM_PER_THREAD]) {
  if (VEC4) {
#pragma unroll
    for (int q = 0; q < UM_PER_THREAD / 4; ++q) {
      const f32x4 val = *reinterpret_cast<const f32x4*>(row + chunk_index<true>(v0, 4 * q));
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = val[e];
    }
  } else {
#pragma unroll
    for (int k = 0; k < UM_PER_THREAD; ++k) x[k] = row[chunk_index<false>(v0, k)];
  }
}
// The row's last chunk when it is ragged: entries past V read as -inf.
template <bool VEC4>
__device__ __forceinline__ void chunk_load_tail(const float* __restrict__ row, int v0, int V,
                                                float (&x)[UM_PER_THREAD]) {
#pragma unroll
  for (int k = 0; k < UM_PER_THREAD; ++k) {
    const int v = chunk_index<VEC4>(v0, k);
    x[k] = (v < V) ? row[v] : -INFINITY;
  }
}

// The loaded chunk reduced by the calling thread and merged into its running record (m, a, s).
template <bool VEC4>
__device__ __forceinline__ void chunk_reduce(float (&x)[UM_PER_THREAD], int v0, int mask_id, float cs, float& m,
                                             int& a, float& s) {
  // the mask token never competes; indices grow with k, so a strict '>' keeps the lowest index
  float mc = -INFINITY;
  int ac = INT32_MAX;
#pragma unroll
  for (int k = 0; k < UM_PER_THREAD; ++k) {
    const int v = chunk_index<VEC4>(v0, k);
    if (v == mask_id) x[k] = -INFINITY;
    if (x[k] > mc) {
      mc = x[k];
      ac = v;
    }
  }
  if (mc == -INFINITY) return;
  float sc = 0.f;
  const float mb = mc * cs;
#pragma unroll
  for (int k = 0; k < UM_PER_THREAD; ++k) sc += tt_exp2(fmaf(x[k], cs, -mb));
  merge(m, a, s, mc, ac, sc, cs);
}

// Chunks [c0, c1) of one row reduced into the thread's record: the whole chunks two at a time,
// the next chunk's loads in flight while the current one is reduced, then the ragged last chunk
// of the row if the range holds it.
template <bool VEC4>
__device__ __forceinline__ void range_reduce(const float* __restrict__ row, int c0, int c1, int V, int mask_id,
                                             float cs, float& m, int& a, float& s) {
  const int cf = min(c1, V / UM_CHUNK);  // chunks [c0, cf) are whole
  float xa[UM_PER_THREAD], xb[UM_PER_THREAD];
  if (c0 < cf) {
    chunk_load<VEC4>(row, c0 * UM_CHUNK, xa);
    int c = c0;
    for (; c + 1 < cf; c += 2) {
      chunk_load<VEC4>(row, (c + 1) * UM_CHUNK, xb);
      chunk_reduce<VEC4>(xa, c * UM_CHUNK, mask_id, cs, m, a, s);
      if (c + 2 < cf) chunk_load<VEC4>(row, (c + 2) * UM_CHUNK, xa);
      chunk_reduce<VEC4>(xb, (c + 1) * UM_CHUNK, mask_id, cs, m, a, s);
    }
    if (c < cf) chunk_reduce<VEC4>(xa, c * UM_CHUNK, mask_id, cs, m, a, s);
  }
  if (max(c0, cf) < c1) {
    chunk_load_tail<VEC4>(row, max(c0, cf) * UM_CHUNK, V, xa);
    chunk_reduce<VEC4>(xa, max(c0, cf) * UM_CHUNK, mask_id, cs, m, a, s);
  }
}

// Merge of the n records p[0..n) into *out by the workgroup: thread t takes records t, t + 256,
// ... in increasing order, then the workgroup merges in a fixed order. PUBLISHED: the records
// were stored by other workgroups of this launch (read with load_record).
constexpr int RM_BATCH = 4;
template <bool PUBLISHED>
__device__ void row_merge(const Partial* __restrict__ p, int n, Partial* __restrict__ out, float cs) {
  float m = -INFINITY, s = 0.f;
  int a = INT32_MAX;
  for (int c0 = threadIdx.x; c0 < n; c0 += UM_THREADS * RM_BATCH) {
    Partial x[RM_BATCH];
#pragma unroll
    for (int k = 0; k < RM_BATCH; ++k) {
      const int c = c0 + UM_THREADS * k;
      if (c < n) x[k] = PUBLISHED ? load_record(p + c) : p[c];
      else x[k] = Partial{-INFINITY, 0.f, INT32_MAX, 0};
    }
#pragma unroll
    for (int k = 0; k < RM_BATCH; ++k) merge(m, a, s, x[k].m, x[k].a, x[k].s, cs);
  }
  wg_merge_store(m, a, s, out, cs);
}

// Commit of block b (mask word `bits` at entry) from the S row records rec[0..S) by the first
// wave of the workgroup: lane i holds position i's confidence and prediction and applies the
// commit rule for the block:
//   kind TT_SAMPLER_CONFIDENCE: conf >= gamma, topped up to the completion floor;
//   kind TT_SAMPLER_PREDICT_NOISE: the n_masked - floor(S (T-1-step) / T) most confident.
__device__ void commit_block(const Partial* __restrict__ rec, int32_t* __restrict__ tokens,
                             uint64_t* __restrict__ mask_bits, int32_t* __restrict__ n_masked,
                             float* __restrict__ conf_out, int32_t* __restrict__ pred_out, int S,
                             int step, int num_steps, int kind, float gamma, int b, uint64_t bits) {
  if (threadIdx.x >= TT_WAVE) return;
  const int i = threadIdx.x;
  const bool masked = (i < S) && ((bits >> i) & 1ull);
  float conf = -1.f;
  int pred = -1;
  if (masked) {
    const Partial x = load_record(rec + i);
    conf = 1.f / x.s;
    pred = x.a;
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
        const bool mj = (mk >> j) & 1ull;
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

// The arrival ticket of a workgroup on counter *cnt (shared by `total` workgroups). Thread 0,
// which stored the workgroup's record with store_record, waits until that store has completed
// (it is then visible to every agent-scope load) and only then takes a ticket, so the workgroup
// that takes the last one finds every record with load_record; that workgroup resets the
// counter to zero (no other workgroup touches it again in this launch) and returns true. The
// counter must be zero when the first workgroup arrives.
__device__ __forceinline__ bool last_arrival(unsigned* cnt, unsigned total) {
  __shared__ int is_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    tt_wait_vmem<0>();
    const bool last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = last;
  }
  __syncthreads();
  return is_last;
}

// The unmasking step (see the top of the file). Grid = B * S * nsplit workgroups; workgroup
// (r, j) reduces chunks [j * cpw, min((j + 1) * cpw, nchunk)) of row r. blk_cnt / row_cnt: B / B*S
// counters, UM_SLOT apart; split_rec [B*S][nsplit] (unused when nsplit == 1); row_rec [B*S].
template <bool VEC4>
__global__ __launch_bounds__(UM_THREADS) void unmask_step(
    const float* __restrict__ logits, int32_t* __restrict__ tokens, uint64_t* __restrict__ mask_bits,
    int32_t* __restrict__ n_masked, float* __restrict__ conf_out, int32_t* __restrict__ pred_out,
    unsigned* __restrict__ blk_cnt, unsigned* __restrict__ row_cnt, Partial* __restrict__ split_rec,
    Partial* __restrict__ row_rec, int S, int V, int nchunk, int nsplit, int cpw, int mask_id, int step,
    int num_steps, int kind, float gamma, float cs) {
  const int r = blockIdx.x / nsplit, j = blockIdx.x - r * nsplit;
  const int b = r / S, i = r - b * S;
  const uint64_t bits = mask_bits[b];
  const bool masked = (bits >> i) & 1ull;
  if (masked) {
    float m = -INFINITY, s = 0.f;
    int a = INT32_MAX;
    const float* row = logits + (size_t)r * V;
    range_reduce<VEC4>(row, j * cpw, min(nchunk, (j + 1) * cpw), V, mask_id, cs, m, a, s);
    wg_merge_store(m, a, s, nsplit > 1 ? split_rec + (size_t)r * nsplit + j : row_rec + r, cs);
  }
  if (nsplit > 1) {
    if (!last_arrival(row_cnt + (size_t)r * UM_SLOT, (unsigned)nsplit)) return;
    if (masked) row_merge<true>(split_rec + (size_t)r * nsplit, nsplit, row_rec + r, cs);
  }
  if (!last_arrival(blk_cnt + (size_t)b * UM_SLOT, (unsigned)S)) return;
  commit_block(row_rec + (size_t)b * S, tokens, mask_bits, n_masked, conf_out, pred_out, S, step, num_steps,
               kind, gamma, b, bits);
}

// The fused path's last kernel: one workgroup per (block, position) merges the row's nparts
// records (stored by the LM-head kernel), then the block's last-arriving row commits it.
__global__ __launch_bounds__(UM_THREADS) void unmask_rowstep(
    const Partial* __restrict__ parts, Partial* __restrict__ rowres, int32_t* __restrict__ tokens,
    uint64_t* __restrict__ mask_bits, int32_t* __restrict__ n_masked, float* __restrict__ conf_out,
    int32_t* __restrict__ pred_out, unsigned* __restrict__ blk_cnt, int S, int nparts, int step,
    int num_steps, int kind, float gamma, float cs) {
  const int r = blockIdx.x;
  const int b = r / S, i = r - b * S;
  const uint64_t bits = mask_bits[b];
  if ((bits >> i) & 1ull) row_merge<false>(parts + (size_t)r * nparts, nparts, rowres + r, cs);
  if (!last_arrival(blk_cnt + (size_t)b * UM_SLOT, (unsigned)S)) return;
  commit_block(rowres + (size_t)b * S, tokens, mask_bits, n_masked, conf_out, pred_out, S, step, num_steps,
               kind, gamma, b, bits);
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

// Arrival counters of B blocks and B*S rows, UM_SLOT apart: the first unmask_counter_bytes(B, S)
// bytes of every unmasking workspace (zero between calls).
size_t unmask_counter_bytes(int B, int S) {
  return tt_align_up(((size_t)B + (size_t)B * S) * UM_SLOT_BYTES, 256);
}

// How unmask_step splits the rows: nsplit workgroups per row, cpw chunks each.
struct UmPlan {
  int nchunk, nsplit, cpw;
  size_t split_bytes, row_bytes;  // record arrays
};
UmPlan unmask_plan(int B, int S, int V) {
  UmPlan p;
  const size_t M = (size_t)B * S;
  p.nchunk = (V + UM_CHUNK - 1) / UM_CHUNK;
  const size_t want = (UM_TARGET_WG + M - 1) / M;
  const int ns = (int)std::min<size_t>(std::max<size_t>(want, 1), (size_t)p.nchunk);
  p.cpw = (p.nchunk + ns - 1) / ns;
  p.nsplit = (p.nchunk + p.cpw - 1) / p.cpw;
  p.split_bytes = p.nsplit > 1 ? M * p.nsplit * sizeof(Partial) : 0;
  p.row_bytes = M * sizeof(Partial);
  return p;
}
size_t unmask_ws_bytes(int B, int S, int V) {
  const UmPlan p = unmask_plan(B, S, V);
  return unmask_counter_bytes(B, S) + p.split_bytes + p.row_bytes;
}

// The unmasking step with its counters at `counters` (B + B*S slots, all zero) and its records at
// `recs` (split_bytes + row_bytes of unmask_plan); arguments already checked.
int unmask_launch(const float* logits, int32_t* tokens, uint64_t* mask_bits, int32_t* n_masked,
                  float* conf_out, int32_t* pred_out, int B, int S, int V, int step, int num_steps,
                  const tt_sampler* sampler, int mask_id, unsigned* counters, void* recs, hipStream_t s) {
  const UmPlan p = unmask_plan(B, S, V);
  const size_t rows = (size_t)B * S;
  const float cs = sampler_scale(sampler);
  unsigned* blk_cnt = counters;
  unsigned* row_cnt = counters + (size_t)B * UM_SLOT;
  Partial* split_rec = (Partial*)recs;
  Partial* row_rec = (Partial*)((char*)recs + p.split_bytes);
  const bool vec4 = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0);
  const dim3 grid((unsigned)(rows * p.nsplit));
  if (vec4)
    hipLaunchKernelGGL(unmask_step<true>, grid, dim3(UM_THREADS), 0, s, logits, tokens, mask_bits, n_masked,
                       conf_out, pred_out, blk_cnt, row_cnt, split_rec, row_rec, S, V, p.nchunk, p.nsplit, p.cpw,
                       mask_id, step, num_steps, sampler->kind, sampler->gamma, cs);
  else
    hipLaunchKernelGGL(unmask_step<false>, grid, dim3(UM_THREADS), 0, s, logits, tokens, mask_bits, n_masked,
                       conf_out, pred_out, blk_cnt, row_cnt, split_rec, row_rec, S, V, p.nchunk, p.nsplit, p.cpw,
                       mask_id, step, num_steps, sampler->kind, sampler->gamma, cs);
  return tt_launch_status();
}

// Scratch of tt_confidence_unmask_noalloc in a fixed array of each device (every GPU the library
// runs on holds it until the process ends): counters in its first UM_SCRATCH_CNT bytes, records
// after them. The array is zero when the code object is loaded and every call leaves its counters
// zero, whatever the sizes of the calls before it. Host code never uses the array's name as an
// address: the device address is looked up once per device.
constexpr size_t UM_SCRATCH_BYTES = (size_t)2 << 20;
constexpr size_t UM_SCRATCH_CNT = (size_t)512 << 10;  // 8192 counter slots
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
  if (S > 64 || V > INT32_MAX - UM_CHUNK) return TT_ERR_UNSUPPORTED;  // chunk indices stay in int
  if ((size_t)B * S * unmask_plan(B, S, V).nsplit > (size_t)INT32_MAX) return TT_ERR_UNSUPPORTED;
  st = tt_workspace_check(workspace, workspace_bytes, unmask_ws_bytes(B, S, V));
  if (st != 0) return st < 0 ? st : TT_OK;
  if ((uintptr_t)workspace % 256) return TT_ERR_ARG;
  return unmask_launch(logits, tokens, mask_bits, n_masked, conf_out, pred_out, B, S, V, step, num_steps,
                       sampler, mask_id, (unsigned*)workspace, (char*)workspace + unmask_counter_bytes(B, S),
                       (hipStream_t)stream);
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
  if (S > 64 || V > INT32_MAX - UM_CHUNK) return TT_ERR_UNSUPPORTED;
  const UmPlan p = unmask_plan(B, S, V);
  if (((size_t)B + (size_t)B * S) * UM_SLOT_BYTES > UM_SCRATCH_CNT ||
      p.split_bytes + p.row_bytes > UM_SCRATCH_BYTES - UM_SCRATCH_CNT)
    return TT_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return TT_ERR_HIP;
  return unmask_launch(logits, tokens, mask_bits, n_masked, conf_out, pred_out, B, S, V, step, num_steps, &sm,
                       mask_id, (unsigned*)ws, (char*)ws + UM_SCRATCH_CNT, (hipStream_t)stream);
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
  // workspace: the arrival counters (zero between calls; only the B block counters are used here),
  // the records, one merged record per row
  const size_t cnt_bytes = unmask_counter_bytes(B, S);
  const size_t parts_bytes = (size_t)M * nparts * sizeof(Partial);
  const size_t need = cnt_bytes + parts_bytes + (size_t)M * sizeof(Partial);
  st = tt_workspace_check(workspace, workspace_bytes, need);
  if (st != 0) return st < 0 ? st : TT_OK;
  if ((uintptr_t)workspace % 256) return TT_ERR_ARG;
  if ((uintptr_t)hidden % 16 || (uintptr_t)w % 16) return TT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  unsigned* counters = (unsigned*)workspace;
  Partial* parts = (Partial*)((char*)workspace + cnt_bytes);
  Partial* rowres = (Partial*)((char*)workspace + cnt_bytes + parts_bytes);
  const float cs = sampler_scale(sampler);
  const TtRedArgs red{bias_tok, bias_val, mask_id, parts, nparts, mask_bits, S, B, cs};
  if (tt_lm_reduce_launch(hidden, w, M, H, V, red, s) != TT_OK) return TT_ERR_HIP;
  hipLaunchKernelGGL(unmask_rowstep, dim3((unsigned)M), dim3(UM_THREADS), 0, s, parts, rowres, tokens, mask_bits,
                     n_masked, conf_out, pred_out, counters, S, nparts, step, num_steps, sampler->kind,
                     sampler->gamma, cs);
  return tt_launch_status();
}
