// LM-head product logits = hidden . W^T ("Nemotron-Labs-TwoTower" wiki page, section "Block-wise
// generation": every denoising step predicts all masked positions of the block in parallel).
//
// hidden [M][H], W [V][H] (dtype), logits [M][V] fp32. At the block step's shapes (M = B*S rows,
// H = 2688, V = 131072) W is 705 MB and is read exactly once; the product is HBM-bound unless M
// reaches a few hundred rows.
//
// Workgroup = 4 waves; each wave owns VT vocabulary tiles (NV rows each) and all MB = MT*BMT
// hidden rows of the workgroup, so each W byte feeds exactly one wave: W fragments go straight
// from HBM into a ring of registers RING pipeline steps (STEP values of h each) ahead of the
// MFMAs. The hidden rows are shared by the 4 waves and staged through LDS in double-buffered
// chunks of KCH columns. Tiles compute C[m][v] with W as the MFMA B operand, so result lanes
// walk consecutive vocabulary ids and the fp32 stores are coalesced.
//
// Reduction order: inside a pipeline step the LPR lanes that share a W row split the STEP
// columns into LPR contiguous spans, lane part p holding h = base + p*STEP/LPR + EPL*ks + i for
// MFMA k-step ks. Each lane therefore reads one contiguous span of its W row per step (its 16-byte
// loads walk consecutive addresses), and the hidden fragments read from LDS use the same order.
//
// When M needs several hidden-row blocks, the workgroups of one vocabulary tile are placed on the
// same XCD (dispatch ids congruent modulo 8 land on the same XCD), so the blocks share W in L2.
#include "lmhead_int.h"
#include "reduce_int.h"

namespace {

constexpr int LM_THREADS = 256;
constexpr int LM_WAVES = 4;
constexpr int NXCD = 8;

// MFMA shapes. Result layout (per lane l, register j):
//   32x32: column l%32, row 8(j/4) + 4(l/32) + j%4 (16 registers)
//   16x16: column l%16, row 4(l/16) + j            (4 registers)
template <typename T, int MT>
struct Shape;

template <>
struct Shape<bf16, 32> {  // v_mfma_f32_32x32x16_bf16
  static constexpr int NV = 32, LPR = 2, EPL = 8, NREG = 16;
  typedef bf16x8 frag;
  typedef f32x16 acc;
  __device__ static __forceinline__ acc mma(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ int row(int lane, int j) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }
};

template <>
struct Shape<bf16, 16> {  // v_mfma_f32_16x16x32_bf16
  static constexpr int NV = 16, LPR = 4, NREG = 4;
  [[maybe_unused]] static constexpr int EPL = 8;
  typedef bf16x8 frag;
  typedef f32x4 acc;
  __device__ static __forceinline__ acc mma(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ int row(int lane, int j) { return 4 * (lane >> 4) + j; }
};

template <>
struct Shape<float, 32> {  // v_mfma_f32_32x32x2f32
  static constexpr int NV = 32, LPR = 2, EPL = 1, NREG = 16;
  typedef float frag;
  typedef f32x16 acc;
  __device__ static __forceinline__ acc mma(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ int row(int lane, int j) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }
};

template <typename F>
__device__ __forceinline__ F frag_zero() {
  F f;
  if constexpr (sizeof(F) == 4) {
    f = 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(F) / 2); ++i) f[i] = (bf16)0.f;
  }
  return f;
}

// T: element type; MT: MFMA rows (hidden rows per tile, 32 or 16); BMT: hidden tiles per
// workgroup; VT: vocabulary tiles per wave; STEP: h per pipeline step; RING: steps in flight;
// KCH: h per LDS chunk of hidden.
template <typename T, int MT, int BMT, int VT, int STEP, int RING, int KCH>
__global__ __launch_bounds__(LM_THREADS) void lmhead_kernel(const T* __restrict__ hidden,
                                                           const T* __restrict__ w,
                                                           float* __restrict__ logits, int M, int H,
                                                           int V, int nvt, int nmb) {
  typedef Shape<T, MT> SH;
  typedef typename SH::frag frag;
  typedef typename SH::acc acc_t;
  constexpr int NV = SH::NV, LPR = SH::LPR, EPL = SH::EPL, NREG = SH::NREG;
  constexpr int KI = LPR * EPL;          // reduction depth of one MFMA
  constexpr int KPS = STEP / KI;         // MFMA k-steps per pipeline step
  constexpr int SPAN = STEP / LPR;       // contiguous h per lane per step
  constexpr int MB = MT * BMT;           // hidden rows per workgroup
  constexpr int BV = LM_WAVES * VT * NV; // vocabulary rows per workgroup
  constexpr int HPAD = 16 / (int)sizeof(T);
  constexpr int HROW = KCH + HPAD;
  constexpr int EV = 16 / (int)sizeof(T);
  constexpr int HVEC = (MB * KCH / EV + LM_THREADS - 1) / LM_THREADS;
  static_assert(STEP % KI == 0 && KCH % STEP == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) T hs[2][MB][HROW];

  const int id = blockIdx.x;
  int vtile, mblk;
  if (nmb == 1) {
    vtile = id;
    mblk = 0;
  } else {
    const int grp = id / (NXCD * nmb);
    const int rem = id - grp * NXCD * nmb;
    mblk = rem / NXCD;
    vtile = grp * NXCD + rem % NXCD;
  }
  if (vtile >= nvt) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane % NV, part = lane / NV;
  const int m0 = mblk * MB;
  const int vbase = vtile * BV + wave * (VT * NV);

  const T* wrow[VT];
  bool wok[VT];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    const int v = vbase + vt * NV + col;
    wok[vt] = v < V;
    wrow[vt] = w + (size_t)(wok[vt] ? v : 0) * H + part * SPAN;
  }

  frag ring[RING][VT][KPS];
  auto wload = [&](frag (&dst)[VT][KPS], int step) {
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int ks = 0; ks < KPS; ++ks) {
        const T* p = wrow[vt] + step * STEP + ks * EPL;
        if (wok[vt]) {  // several lanes/instructions share each W line: plain loads keep it in L2
          if constexpr (EPL == 8) dst[vt][ks] = *reinterpret_cast<const frag*>(p);
          else dst[vt][ks] = *p;
        } else {
          dst[vt][ks] = frag_zero<frag>();
        }
      }
  };
  // hidden chunk: fetched into registers one chunk ahead, stored to LDS at the chunk boundary
  u32x4 hreg[HVEC];
  auto hfetch = [&](int chunk) {
    const int hc0 = chunk * KCH;
#pragma unroll
    for (int i = 0; i < HVEC; ++i) {
      const int v = tid + LM_THREADS * i;
      const int r = v / (KCH / EV), piece = v % (KCH / EV);
      const int m = m0 + r, h = hc0 + piece * EV;
      hreg[i] = (r < MB && m < M && h < H) ? *reinterpret_cast<const u32x4*>(hidden + (size_t)m * H + h)
                                          : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto hstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < HVEC; ++i) {
      const int v = tid + LM_THREADS * i;
      const int r = v / (KCH / EV), piece = v % (KCH / EV);
      if (r < MB) *reinterpret_cast<u32x4*>(&hs[buf][r][piece * EV]) = hreg[i];
    }
  };

  acc_t acc[BMT][VT];
#pragma unroll
  for (int mt = 0; mt < BMT; ++mt)
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int j = 0; j < NREG; ++j) acc[mt][vt][j] = 0.f;

  const int nsteps = H / STEP;
  const int nchunk = (H + KCH - 1) / KCH;
  constexpr int SPC = KCH / STEP;  // steps per chunk
#pragma unroll
  for (int r = 0; r < RING; ++r)
    if (r < nsteps) wload(ring[r], r);
  hfetch(0);
  hstore(0);
  __syncthreads();

  for (int s0 = 0; s0 < nsteps; s0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int s = s0 + r;
      if (s < nsteps) {
        const int chunk = s / SPC, sc = s - chunk * SPC;
        const int buf = chunk & 1;
        if (sc == 0 && chunk + 1 < nchunk) hfetch(chunk + 1);
#pragma unroll
        for (int ks = 0; ks < KPS; ++ks) {
#pragma unroll
          for (int mt = 0; mt < BMT; ++mt) {
            frag a;
            const int hcol = sc * STEP + part * SPAN + ks * EPL;
            if constexpr (EPL == 8) a = *reinterpret_cast<const frag*>(&hs[buf][mt * MT + col % MT][hcol]);
            else a = hs[buf][mt * MT + col % MT][hcol];
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) acc[mt][vt] = SH::mma(a, ring[r][vt][ks], acc[mt][vt]);
          }
        }
        if (s + RING < nsteps) wload(ring[r], s + RING);
        if (sc == SPC - 1 || s == nsteps - 1) {  // chunk boundary: publish the next hidden chunk
          if (chunk + 1 < nchunk) hstore(buf ^ 1);
          tt_lds_barrier();
        }
      }
    }
  }

#pragma unroll
  for (int mt = 0; mt < BMT; ++mt)
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      const int v = vbase + vt * NV + col;
      if (v >= V) continue;
#pragma unroll
      for (int j = 0; j < NREG; ++j) {
        const int m = m0 + mt * MT + SH::row(lane, j);
        if (m < M) logits[(size_t)m * V + v] = acc[mt][vt][j];
      }
    }
}

template <typename T, int MT, int BMT, int VT, int STEP, int RING, int KCH>
int lm_launch(const void* hidden, const void* w, float* logits, int M, int H, int V, hipStream_t s) {
  constexpr int BV = LM_WAVES * VT * Shape<T, MT>::NV;
  const int nvt = (V + BV - 1) / BV;
  const int nmb = (M + MT * BMT - 1) / (MT * BMT);
  unsigned grid;
  if (nmb == 1) grid = (unsigned)nvt;
  else grid = (unsigned)(((nvt + NXCD - 1) / NXCD) * NXCD * nmb);
  hipLaunchKernelGGL((lmhead_kernel<T, MT, BMT, VT, STEP, RING, KCH>), dim3(grid), dim3(LM_THREADS), 0, s,
                     (const T*)hidden, (const T*)w, logits, M, H, V, nvt, nmb);
  return tt_launch_status();
}


// LDS-staged variant: W is read with whole-line coalesced 16-byte loads (consecutive lanes walk a
// row; each 128-byte line is consumed by one instruction, so non-temporal loads are safe), staged
// through LDS, and read back in MFMA operand layout. Workgroup = 4 waves x (VT tiles of NV rows);
// each stage covers KW columns of h for the TV vocabulary rows and the MB hidden rows of the
// workgroup. NSET register sets keep up to NSET stages of global loads in flight; LDS is double
// buffered, so one barrier per stage separates the writes of stage g+1 from the reads of stage g.
// RED = true: instead of storing logits, reduce each row over the wave's VT * NV columns to one
// (max, lowest argmax, sum exp) record in red.parts[row][vtile * LM_WAVES + wave].
template <int MT, int BMT, int VT, int KW, bool NT, int NSET, bool RED = false>
__global__ __launch_bounds__(LM_THREADS) void lmhead_lds_kernel(const bf16* __restrict__ hidden,
                                                               const bf16* __restrict__ w,
                                                               float* __restrict__ logits, int M, int H,
                                                               int V, int nvt, int nmb, TtRedArgs red) {
  typedef Shape<bf16, MT> SH;
  typedef typename SH::frag frag;
  typedef typename SH::acc acc_t;
  constexpr int NV = SH::NV, LPR = SH::LPR, NREG = SH::NREG;
  constexpr int KI = LPR * 8;             // reduction depth of one MFMA
  constexpr int MB = MT * BMT;
  constexpr int TV = LM_WAVES * VT * NV;   // vocabulary rows per workgroup
  constexpr int ROW = KW + 8;              // LDS row (elements): 16-byte pad staggers banks
  constexpr int VPR = KW / 8;              // 16-byte vectors per row per stage
  constexpr int NWV = TV * VPR / LM_THREADS;
  constexpr int NHV = (MB * VPR + LM_THREADS - 1) / LM_THREADS;
  static_assert(TV * VPR % LM_THREADS == 0 && KW % KI == 0 && NSET % 2 == 0, "stage shape");
  __shared__ __attribute__((aligned(16))) bf16 wsm[2][TV][ROW];
  __shared__ __attribute__((aligned(16))) bf16 hsm[2][MB][ROW];

  const int id = blockIdx.x;
  int vtile, mblk;
  if (nmb == 1) {
    vtile = id;
    mblk = 0;
  } else {
    const int grp = id / (NXCD * nmb);
    const int rem = id - grp * NXCD * nmb;
    mblk = rem / NXCD;
    vtile = grp * NXCD + rem % NXCD;
  }
  if (vtile >= nvt) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane % NV, part = lane / NV;
  const int m0 = mblk * MB, v0 = vtile * TV;

  u32x4 wr[NSET][NWV], hr[NSET][NHV];
  auto gload = [&](int set, int st) {
    const int h0 = st * KW;
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const int v = tid + LM_THREADS * i;
      const int r = v / VPR, pc = v % VPR;
      const int vv = v0 + r;
      const bf16* p = w + (size_t)vv * H + h0 + pc * 8;
      if (vv < V) wr[set][i] = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))
                                  : *reinterpret_cast<const u32x4*>(p);
      else wr[set][i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < NHV; ++i) {
      const int v = tid + LM_THREADS * i;
      const int r = v / VPR, pc = v % VPR;
      const int m = m0 + r;
      hr[set][i] = (r < MB && m < M) ? *reinterpret_cast<const u32x4*>(hidden + (size_t)m * H + h0 + pc * 8)
                                     : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const int v = tid + LM_THREADS * i;
      *reinterpret_cast<u32x4*>(&wsm[buf][v / VPR][(v % VPR) * 8]) = wr[set][i];
    }
#pragma unroll
    for (int i = 0; i < NHV; ++i) {
      const int v = tid + LM_THREADS * i;
      if (v / VPR < MB) *reinterpret_cast<u32x4*>(&hsm[buf][v / VPR][(v % VPR) * 8]) = hr[set][i];
    }
  };

  acc_t acc[BMT][VT];
#pragma unroll
  for (int mt = 0; mt < BMT; ++mt)
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int j = 0; j < NREG; ++j) acc[mt][vt][j] = 0.f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < KW / KI; ++ks) {
      const int hc = ks * KI + part * 8;
      frag b[VT];
#pragma unroll
      for (int vt = 0; vt < VT; ++vt)
        b[vt] = *reinterpret_cast<const frag*>(&wsm[buf][(wave * VT + vt) * NV + col][hc]);
#pragma unroll
      for (int mt = 0; mt < BMT; ++mt) {
        const frag a = *reinterpret_cast<const frag*>(&hsm[buf][mt * MT + col % MT][hc]);
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) acc[mt][vt] = SH::mma(a, b[vt], acc[mt][vt]);
      }
    }
  };

  // stage g lives in register set g % NSET and LDS buffer g % 2; loads run NSET-1 stages ahead
  const int nst = H / KW;
#pragma unroll
  for (int e = 0; e < NSET; ++e)
    if (e < nst) gload(e, e);
  sstore(0, 0);
  __syncthreads();
  for (int g0 = 0; g0 < nst; g0 += NSET) {
#pragma unroll
    for (int e = 0; e < NSET; ++e) {
      const int g = g0 + e;
      if (g < nst) {
        compute(e & 1);
        if (g + 1 < nst) sstore((e + 1) % NSET, (e + 1) & 1);
        if (g + NSET < nst) gload(e, g + NSET);
        tt_lds_barrier();
      }
    }
  }

  if constexpr (RED) {
    // the NV lanes of a group share NREG rows per hidden tile; reduce over their VT * NV columns
    constexpr int W = VT * NV;
    const int cb = v0 + wave * W;
    if (cb >= V) return;
    const int part = vtile * LM_WAVES + wave;
    // wave-uniform choice: only blocks holding the mask id, the vocabulary's end or some row's
    // bias entry need the per-entry checks
    bool slow = (red.mask_id >= cb && red.mask_id < cb + W) || (cb + W > V);
    if (red.bias_tok) {
      bool hit = false;
#pragma unroll
      for (int r = lane; r < MB; r += 64) {
        const int m = m0 + r;
        if (m < M) {
          const int t = red.bias_tok[m];
          hit = hit || (t >= cb && t < cb + W);
        }
      }
      slow = slow || __any(hit);
    }
    auto emit = [&](int m, float rm, int ra, float rs) {
      if (col == 0 && m < M) {
        TtPartial p;
        p.m = rm;
        p.s = rs;
        p.a = ra;
        p.pad = 0;
        red.parts[(size_t)m * red.nparts + part] = p;
      }
    };
    if (!slow) {
#pragma unroll
      for (int mt = 0; mt < BMT; ++mt)
#pragma unroll
        for (int j = 0; j < NREG; ++j) {
          float v[VT];
#pragma unroll
          for (int vt = 0; vt < VT; ++vt) v[vt] = acc[mt][vt][j];
          float rm, rs;
          int ra;
          tt_row_reduce<VT, NV>(v, cb, NV, col, red.c, rm, ra, rs);
          emit(m0 + mt * MT + SH::row(lane, j), rm, ra, rs);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < BMT; ++mt)
#pragma unroll
        for (int j = 0; j < NREG; ++j) {
          const int m = m0 + mt * MT + SH::row(lane, j);
          const int mc = min(m, M - 1);
          const int btok = red.bias_tok ? red.bias_tok[mc] : -1;
          const float bval = red.bias_tok ? red.bias_val[mc] : 0.f;
          float v[VT];
#pragma unroll
          for (int vt = 0; vt < VT; ++vt)
            v[vt] = tt_red_logit(acc[mt][vt][j], cb + vt * NV + col, V, btok, bval, red.mask_id);
          float rm, rs;
          int ra;
          tt_row_reduce<VT, NV>(v, cb, NV, col, red.c, rm, ra, rs);
          emit(m, rm, ra, rs);
        }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < BMT; ++mt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const int v = v0 + (wave * VT + vt) * NV + col;
        if (v >= V) continue;
#pragma unroll
        for (int j = 0; j < NREG; ++j) {
          const int m = m0 + mt * MT + SH::row(lane, j);
          if (m < M) logits[(size_t)m * V + v] = acc[mt][vt][j];
        }
      }
  }
}

template <int MT, int BMT, int VT, int KW, bool NT, int NSET, bool RED = false>
int lm_lds_launch(const void* hidden, const void* w, float* logits, int M, int H, int V, hipStream_t s,
                  TtRedArgs red = TtRedArgs{nullptr, nullptr, -1, nullptr, 0}) {
  constexpr int TV = LM_WAVES * VT * Shape<bf16, MT>::NV;
  const int nvt = (V + TV - 1) / TV;
  const int nmb = (M + MT * BMT - 1) / (MT * BMT);
  unsigned grid;
  if (nmb == 1) grid = (unsigned)nvt;
  else grid = (unsigned)(((nvt + NXCD - 1) / NXCD) * NXCD * nmb);
  hipLaunchKernelGGL((lmhead_lds_kernel<MT, BMT, VT, KW, NT, NSET, RED>), dim3(grid), dim3(LM_THREADS), 0, s,
                     (const bf16*)hidden, (const bf16*)w, logits, M, H, V, nvt, nmb, red);
  return tt_launch_status();
}

// columns of one wave's reduction record in the fused path of an LDS-kernel configuration
template <int MT, int BMT, int VT, int KW, bool NT, int NSET>
constexpr int lds_cols_per_part() { return VT * Shape<bf16, MT>::NV; }

// Kernel choice (measured on MI355X at H = 2688, V = 131072): M <= 16 the LDS-staged kernel
// <MT, BMT, VT, KW, NT, NSET>; larger M the MFMA GEMM kernel (gemm.hip), which with its
// non-temporal W stream beats the LDS-staged kernel from 17 rows on (123 against 137 us at 64
// rows) while its grid fills the chip (lm_use_lds below has the small-vocabulary exception);
// the direct kernel <MT, BMT, VT, STEP, RING, KCH> for fp32 and for H not a multiple of the
// stage width.
#ifndef TT_LM_LDS16
#define TT_LM_LDS16 16, 1, 4, 64, true, 4
#endif
#ifndef TT_LM_CFG32
#define TT_LM_CFG32 32, 1, 2, 32, 8, 256
#endif
#ifndef TT_LM_CFG64
#define TT_LM_CFG64 32, 2, 2, 32, 8, 256
#endif
#ifndef TT_LM_CFGBIG
#define TT_LM_CFGBIG 32, 4, 2, 32, 8, 256
#endif

template <int MT, int BMT, int VT, int STEP, int RING, int KCH>
int lm_direct(const void* h, const void* w, float* o, int M, int H, int V, hipStream_t s) {
  if (H % STEP != 0) return lm_launch<bf16, MT, BMT, VT, 32, RING * STEP / 32, KCH>(h, w, o, M, H, V, s);
  return lm_launch<bf16, MT, BMT, VT, STEP, RING, KCH>(h, w, o, M, H, V, s);
}

// The LDS-staged kernel's vocabulary tile follows the grid: the widest tile (64 VT rows per wave,
// VT = 4, 2, 1) whose vocabulary tiles times 16-row blocks still give 512 workgroups (two per
// compute unit), else the narrowest. At V = 131072 and up to 16 rows that is VT = 4. A small
// vocabulary, such as one GPU's shard of a split LM head, stays spread over the chip. Measured at
// H = 2688, 16 rows: V = 16384 takes 31.6 us with VT = 1 against 44.3 us with VT = 4, V = 32768
// 36.2 against 46.8 us; V = 131072 stays with VT = 4 (106.8 against 118.2 us with VT = 1). Every
// logit is the same chain of MFMAs for any VT, so the values do not depend on the choice.
int lds_vt(int M, int V) {
  const int nmb = (M + 15) / 16;
  if ((int64_t)((V + 255) / 256) * nmb >= 512) return 4;
  if ((int64_t)((V + 127) / 128) * nmb >= 512) return 2;
  return 1;
}

// bf16 with H a multiple of the LDS stage: the LDS-staged kernel up to 16 rows, and up to 128 rows
// when the GEMM kernel's 128 x 512 tiles would give 64 workgroups or fewer (V <= 32768) and the
// LDS-staged kernel's re-reads of W (one per 16 rows) stay small (V M <= 2^21). With so few
// workgroups one workgroup's pass over H sets the GEMM's time whatever M: about 91 us at
// V = 16384, against 32-37 us for the LDS-staged kernel at 32-64 rows and 63 us at 128 rows
// (measured at H = 2688).
bool lm_use_lds(int M, int H, int V) {
  if (H % 64 != 0) return false;
  return M <= 16 || (M <= 128 && (V + 511) / 512 <= 64 && (int64_t)V * M <= (int64_t)1 << 21);
}

template <bool RED>
int lm_lds_by_vt(const void* h, const void* w, float* o, int M, int H, int V, hipStream_t s, TtRedArgs red) {
  const int vt = lds_vt(M, V);
  static_assert(LM_WAVES * lds_cols_per_part<TT_LM_LDS16>() == 256, "VT = 4 is the 256-row tile");
  if (vt == 4) return lm_lds_launch<TT_LM_LDS16, RED>(h, w, o, M, H, V, s, red);
  if (vt == 2) return lm_lds_launch<16, 1, 2, 64, true, 4, RED>(h, w, o, M, H, V, s, red);
  return lm_lds_launch<16, 1, 1, 64, true, 4, RED>(h, w, o, M, H, V, s, red);
}

int lm_bf16(const void* h, const void* w, float* o, int M, int H, int V, hipStream_t s) {
  const TtRedArgs none{nullptr, nullptr, -1, nullptr, 0};
  if (lm_use_lds(M, H, V)) return lm_lds_by_vt<false>(h, w, o, M, H, V, s, none);
  if (M > 16 && H % TT_GEMM_KB == 0) return tt_lm_gemm_launch(h, w, o, M, H, V, s);
  if (M <= 32) return lm_direct<TT_LM_CFG32>(h, w, o, M, H, V, s);
  if (M <= 64) return lm_direct<TT_LM_CFG64>(h, w, o, M, H, V, s);
  return lm_direct<TT_LM_CFGBIG>(h, w, o, M, H, V, s);
}

}  // namespace

// Fused LM head + vocabulary reduction (bf16, H % 64 == 0): which kernel, and how many records per
// row it writes. The same kernel as the logits path for each (M, V), so the accumulators are the
// same: the LDS-staged kernel (16 VT columns per record) where lm_use_lds holds, else the GEMM
// kernel (64 or 128 columns per record, by its tile).
int tt_lm_reduce_nparts(int M, int H, int V) {
  const int cols = lm_use_lds(M, H, V) ? 16 * lds_vt(M, V) : tt_lm_gemm_cols(M, V);
  return (V + cols - 1) / cols;
}

int tt_lm_reduce_launch(const void* hidden, const void* w, int M, int H, int V, TtRedArgs red, hipStream_t s) {
  if (lm_use_lds(M, H, V)) return lm_lds_by_vt<true>(hidden, w, nullptr, M, H, V, s, red);
  return tt_lm_gemm_reduce_launch(hidden, w, M, H, V, red, s);
}

extern "C" int tt_lmhead_logits(const void* hidden, const void* w, float* logits, int M, int H,
                                int V, int dtype, void* stream) {
  if (!hidden || !w || !logits) return TT_ERR_ARG;
  if (M <= 0 || H <= 0 || V <= 0) return TT_ERR_ARG;
  if (dtype != TT_F32 && dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (H % 32 != 0) return TT_ERR_UNSUPPORTED;
  if ((uintptr_t)hidden % 16 || (uintptr_t)w % 16) return TT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == TT_BF16) return lm_bf16(hidden, w, logits, M, H, V, s);
  if (M <= 32) return lm_launch<float, 32, 1, 2, 32, 2, 64>(hidden, w, logits, M, H, V, s);
  return lm_launch<float, 32, 4, 2, 32, 2, 64>(hidden, w, logits, M, H, V, s);
}
