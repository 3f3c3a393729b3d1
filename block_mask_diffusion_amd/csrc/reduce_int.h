// Internal: the vocabulary-reduction record shared by the unmask kernels and the fused LM-head
// epilogue (not part of the C ABI).
#pragma once

#include "common.h"

// (max, lowest argmax, sum of exp((l - max) / temperature)) of a set of logits of one row; m =
// -inf and a = INT32_MAX for an empty set. The sums of one call share the scale c =
// log2(e) / temperature: s = sum exp2((l - m) c).
struct alignas(16) TtPartial {
  float m;
  float s;
  int a;
  int pad;
};

constexpr float TT_LOG2E = 1.4426950408889634f;

// Merge (m2, a2, s2) into (m, a, s) at scale c; ties of the max keep the lower index.
__device__ __forceinline__ void tt_merge(float& m, int& a, float& s, float m2, int a2, float s2, float c) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;  // both empty
  const float t1 = (m == -INFINITY) ? 0.f : s * tt_exp2((m - M) * c);
  const float t2 = (m2 == -INFINITY) ? 0.f : s2 * tt_exp2((m2 - M) * c);
  const int an = (m2 > m) ? a2 : ((m > m2) ? a : min(a, a2));
  m = M;
  a = an;
  s = t1 + t2;
}

// Arguments of the fused LM-head + vocabulary-reduction epilogue.
struct TtRedArgs {
  const int32_t* bias_tok;  // [M] vocabulary id of each row's additive bias, or NULL
  const float* bias_val;    // [M] its value
  int mask_id;              // never a candidate (its logit counts as -inf)
  TtPartial* parts;         // [M][nparts]: one record per (row, column block of one wave)
  int nparts;
  // optional: only rows b * S + i with bit i of mask_bits[b] set need a record (kernels that
  // can skip the other rows do; NULL = every row)
  const uint64_t* mask_bits;
  int S, B;
  float c;                  // log2(e) / temperature
};

// Cross-lane partner values for a butterfly over groups of up to 32 consecutive lanes, all on
// the VALU (DPP and v_permlane16_swap; no LDS round trip). Level 0 pairs lanes l and l ^ 1,
// level 1 l and l ^ 2 (quad permutes); level 2 mirrors each half row of 8 lanes, level 3 each
// row of 16, level 4 swaps rows 2r and 2r + 1. After levels 0..L-1 every lane of an aligned
// group of 2^L lanes has combined all of the group's values (each level joins two halves that
// are already reduced), which is all a commutative reduction needs.
template <int CTRL>
__device__ __forceinline__ int tt_dpp(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);  // every source lane exists
}
template <int LVL>
__device__ __forceinline__ int tt_partner(int x) {
  static_assert(LVL >= 0 && LVL <= 4, "butterfly level");
  if constexpr (LVL == 0) return tt_dpp<0xB1>(x);       // quad_perm [1, 0, 3, 2]
  else if constexpr (LVL == 1) return tt_dpp<0x4E>(x);  // quad_perm [2, 3, 0, 1]
  else if constexpr (LVL == 2) return tt_dpp<0x141>(x); // row_half_mirror
  else if constexpr (LVL == 3) return tt_dpp<0x140>(x); // row_mirror
  else {
    // v_permlane16_swap with both operands x: odd rows find their even neighbour's value in the
    // first result, even rows their odd neighbour's in the second
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    return (int)((threadIdx.x & 16) ? r[0] : r[1]);
  }
}
template <int LVL>
__device__ __forceinline__ float tt_partner(float x) {
  return __int_as_float(tt_partner<LVL>(__float_as_int(x)));
}

template <int NL>
__device__ __forceinline__ float tt_group_max(float x) {
  static_assert(NL == 16 || NL == 32, "group of 16 or 32 lanes");
  x = fmaxf(x, tt_partner<0>(x));
  x = fmaxf(x, tt_partner<1>(x));
  x = fmaxf(x, tt_partner<2>(x));
  x = fmaxf(x, tt_partner<3>(x));
  if constexpr (NL == 32) x = fmaxf(x, tt_partner<4>(x));
  return x;
}
template <int NL>
__device__ __forceinline__ float tt_group_sum(float x) {
  x += tt_partner<0>(x);
  x += tt_partner<1>(x);
  x += tt_partner<2>(x);
  x += tt_partner<3>(x);
  if constexpr (NL == 32) x += tt_partner<4>(x);
  return x;
}
template <int NL>
__device__ __forceinline__ int tt_group_min(int x) {
  x = min(x, tt_partner<0>(x));
  x = min(x, tt_partner<1>(x));
  x = min(x, tt_partner<2>(x));
  x = min(x, tt_partner<3>(x));
  if constexpr (NL == 32) x = min(x, tt_partner<4>(x));
  return x;
}

// Row reduction across an aligned group of NL consecutive lanes (16 or 32) that hold the same
// row: lane `col` of the group brings the K logits of vocabulary ids cb + k * stride + col
// (stride >= NL; -inf for excluded entries). Returns, on every lane of the group, the row's
// (max, lowest id attaining it, sum exp2((l - max) c)); an all -inf row gives (-inf, INT32_MAX,
// 0).
template <int K, int NL>
__device__ __forceinline__ void tt_row_reduce(const float (&v)[K], int cb, int stride, int col, float c,
                                              float& M, int& A, float& S) {
  float m = v[0];
#pragma unroll
  for (int k = 1; k < K; ++k) m = fmaxf(m, v[k]);
  m = tt_group_max<NL>(m);
  const bool empty = (m == -INFINITY);
  const float mb = empty ? 0.f : m * c;
  int key = INT32_MAX;  // k * NL + col of this lane's first maximum: ordered like the vocabulary id
#pragma unroll
  for (int k = K - 1; k >= 0; --k) key = (v[k] == m) ? k * NL + col : key;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) s += tt_exp2(fmaf(v[k], c, -mb));
  key = tt_group_min<NL>(key);
  s = tt_group_sum<NL>(s);
  M = m;
  A = empty ? INT32_MAX : cb + (key / NL) * stride + key % NL;
  S = s;
}

// Logit of (row m, vocabulary id v) as the reduction sees it: past V or the mask id -> -inf,
// plus the row's bias when v is its bias id.
__device__ __forceinline__ float tt_red_logit(float x, int v, int V, int btok, float bval, int mask_id) {
  if (v == btok) x += bval;
  return (v >= V || v == mask_id) ? -INFINITY : x;
}
