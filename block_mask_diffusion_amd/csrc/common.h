// Shared types and helpers of the gfx950 kernels behind tt.h.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "tt.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define TT_WAVE 64

static inline size_t tt_align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Map the outcome of a kernel launch to a status code.
static inline int tt_launch_status() {
  return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

// Workspace protocol shared by the calls that take one (see tt.h).
//   returns 1 when the caller only asked for the size (nothing to launch), 0 to proceed,
//   or a negative status.
static inline int tt_workspace_check(void* ws, size_t* ws_bytes, size_t need) {
  if (ws_bytes == nullptr) return TT_ERR_ARG;
  if (ws == nullptr) {
    *ws_bytes = need;
    return 1;
  }
  if (*ws_bytes < need) return TT_ERR_WORKSPACE;
  return 0;
}

// Cross-lane helpers (wave64).
__device__ __forceinline__ float tt_shfl_xor(float v, int mask) { return __shfl_xor(v, mask, TT_WAVE); }
__device__ __forceinline__ int tt_shfl_xor(int v, int mask) { return __shfl_xor(v, mask, TT_WAVE); }

// Value of lane l ^ 32 (the other half of the wave) without an LDS round trip: one
// v_permlane32_swap exchanges the upper half of its first operand with the lower half of its
// second, so with both operands = v, lanes 0..31 find their partner in the second result and
// lanes 32..63 in the first.
__device__ __forceinline__ float tt_swap_halves(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ int tt_swap_halves_i(int v) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return (int)((threadIdx.x & 32) ? r[0] : r[1]);
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1 (a compile-time index for each call)
template <int N, int I = 0, typename F>
__device__ __forceinline__ void tt_static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    tt_static_for<N, I + 1>(f);
  }
}

// Issues fm(i) for i = 0 .. NM-1 and, spread evenly behind them, fl(l) for l = 0 .. NL-1 (LDS
// reads) and fv(e) for e = 0 .. NV-1 (vector arithmetic); every MFMA with its share is pinned in
// that order by a scheduling barrier. A wave's own vector work then issues while its matrix-core
// work runs, instead of waiting for it.
template <int NM, int NV, int NL, typename FM, typename FV, typename FL>
__device__ __forceinline__ void tt_interleave(FM&& fm, FV&& fv, FL&& fl) {
  tt_static_for<NM>([&](auto i) {
    constexpr int I = decltype(i)::value;
    fm(i);
    constexpr int L0 = I * NL / NM, L1 = (I + 1) * NL / NM;
    tt_static_for<L1 - L0>([&](auto k) { fl(std::integral_constant<int, L0 + decltype(k)::value>{}); });
    constexpr int E0 = I * NV / NM, E1 = (I + 1) * NV / NM;
    tt_static_for<E1 - E0>([&](auto k) { fv(std::integral_constant<int, E0 + decltype(k)::value>{}); });
    __builtin_amdgcn_sched_barrier(0);
  });
}

// max(v, v of the lane 32 away): after the half swap one register holds the lower half's values
// in both halves' lanes and the other the upper half's, so their max is the pair max everywhere.
// The max is one v_max_f32 (fmaxf would first quiet both operands, two more instructions; the
// operands here are scores or -inf, never signalling NaNs).
__device__ __forceinline__ float tt_max_halves(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
}

// exp2 on the hardware transcendental unit (v_exp_f32): exact at 0, returns 0 for -inf.
__device__ __forceinline__ float tt_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier for an LDS hand-off: waits for this wave's own LDS operations, then
// s_barrier. Unlike __syncthreads() it does not wait for outstanding global loads, so prefetches
// issued before it stay in flight. The "memory" clobber keeps the compiler from moving memory
// accesses across it; register data of earlier global loads is still waited for where it is used.
__device__ __forceinline__ void tt_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are outstanding (they complete
// in issue order).
template <int N>
__device__ __forceinline__ void tt_wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt immediate for "vmcnt(0)" alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8; the other counters at their maxima)
#define TT_WAIT_VMCNT0 0x0F70
// ... and for "lgkmcnt(0)" alone (vmcnt 63, expcnt 7)
#define TT_WAIT_LGKMCNT0 0xC07F

#define TT_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// A pointer that has the same value in every lane, moved to scalar registers (a scalar operand
// of an instruction needs the compiler to know it is uniform).
template <typename T>
__device__ __forceinline__ T* tt_uniform(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// LDS byte address of a __shared__ location, made wave-uniform (it goes to M0).
__device__ __forceinline__ uint32_t tt_lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)TT_LDS_PTR(const void, p));
}

// Direct global->LDS load of 16 bytes per lane (lane i's bytes land at LDS address base + 16 i),
// with the non-temporal cache policy, for data read exactly once (a streamed KV cache or weight
// matrix): on MI355X a stream of these reaches about 7.1 TB/s from HBM against 6.1 TB/s without
// the policy. Written as inline asm on purpose: the compiler then does not track these writes to
// LDS, so it does not put a wait for every outstanding global load in front of each LDS read of
// a ring that such loads fill. Ordering is the caller's job instead: each stage's readers wait
// (counted vmcnt, then a barrier) for that stage's loads only, and a buffer is refilled only after
// the barrier that ends its reads. M0 (which holds the LDS base) is saved to a scratch SGPR and
// restored inside the same asm, so the compiler's own use of M0 is unaffected. The only register
// output is that scratch SGPR, written by a scalar move; the load returns nothing to registers.
__device__ __forceinline__ void tt_dma16_nt(const void* gptr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"  // one wait state between an SALU write of M0 and its use by an LDS DMA
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_base)
      : "memory");
}

// Direct global->LDS load (non-temporal) from a wave-uniform base plus a per-lane 32-bit byte
// offset (the scalar-base form of the instruction), into LDS at lds_base + OFF + 16 lane. M0 is
// saved and restored inside the asm as in tt_dma16_nt.
template <int OFF>
__device__ __forceinline__ void tt_dma16_snt(uint32_t voff, const void* sbase, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %3, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_base), "i"(OFF)
      : "memory", "scc");
}

// Four direct global->LDS loads (non-temporal), 16 bytes per lane each, from two wave-uniform
// bases plus per-lane 32-bit byte offsets (the scalar-base form of the instruction): load i reads
// sbase[i / 2] + voff[i] and writes LDS at lds_base + OFF_i + 16 lane. One asm block saves M0
// once, sets it before each load (one wait state between an SALU write of M0 and its use) and
// restores it at the end.
template <int OFF0, int OFF1, int OFF2, int OFF3>
__device__ __forceinline__ void tt_dma16x4_snt(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                               const void* sbase0, const void* sbase1,
                                               uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %7, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5 nt\n\t"
      "s_add_u32 m0, %7, %9\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %5 nt\n\t"
      "s_add_u32 m0, %7, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %6 nt\n\t"
      "s_add_u32 m0, %7, %11\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %6 nt\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(sbase0), "s"(sbase1), "s"(lds_base), "i"(OFF0),
        "i"(OFF1), "i"(OFF2), "i"(OFF3)
      : "memory", "scc");
}

// The same with the LDS address given as a base plus a constant byte offset, added into M0 inside
// the asm: a loop that fills many slots from one base keeps a single scalar register live. NT
// selects the non-temporal policy.
template <int OFF, bool NT = false>
__device__ __forceinline__ void tt_dma16_at(const void* gptr, uint32_t lds_base) {
  uint32_t saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_add_u32 m0, %2, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_base), "i"(OFF)
        : "memory", "scc");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_add_u32 m0, %2, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_base), "i"(OFF)
        : "memory", "scc");
  }
}
