// LM-head product logits = hidden . W^T ("Nemotron-Labs-TwoTower" wiki page, section "Block-wise
// generation": every denoising step predicts all masked positions of the block in parallel).
//
// hidden [M][H], W [V][H] (dtype), logits [M][V] fp32. At the block step's shapes (M = B*S rows,
// H = 2688, V = 131072) W is 705 MB and is read exactly once; the product is HBM-bound unless M
// reaches a few hundred rows.
//
// Workgroup = 4 waves = 256 vocabulary rows x (32*BMT) hidden rows. Each wave owns two 32-row
// vocabulary tiles and every hidden row of the workgroup, so each W byte feeds exactly one wave:
// W fragments go straight from HBM into a ring of registers RING steps (of 32 h each) ahead of
// the MFMAs. The hidden rows are shared by the 4 waves and staged through LDS in double-buffered
// chunks of KCH columns. MFMA tiles compute C[m][v] with W as the B operand, so the 32 lanes of a
// result row hold 32 consecutive vocabulary ids and the fp32 stores are 128-byte coalesced.
// When M needs several hidden-row blocks, the workgroups of one vocabulary tile are placed on the
// same XCD (consecutive dispatch ids modulo 8 land on the same XCD), so the blocks share W in L2.
#include "common.h"

namespace {

constexpr int LM_THREADS = 256;
constexpr int LM_WAVES = 4;
constexpr int VT_PER_WAVE = 2;
constexpr int BV = LM_WAVES * VT_PER_WAVE * 32;  // vocabulary rows per workgroup
constexpr int STEP = 32;                          // h per pipeline step
constexpr int NXCD = 8;

template <typename T>
struct Lm;

template <>
struct Lm<bf16> {
  static constexpr int KS = 16, EPL = 8, RING = 8;
  static constexpr int KCH = 256;  // h per LDS chunk of hidden
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)0.f;
    return f;
  }
};

template <>
struct Lm<float> {
  static constexpr int KS = 2, EPL = 1, RING = 2;
  static constexpr int KCH = 64;
  typedef float frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag zero() { return 0.f; }
};

template <typename T, int BMT>
__global__ __launch_bounds__(LM_THREADS, 1) void lmhead_kernel(const T* __restrict__ hidden,
                                                               const T* __restrict__ w,
                                                               float* __restrict__ logits, int M,
                                                               int H, int V, int nvt, int nmb) {
  typedef Lm<T> L;
  typedef typename L::frag frag;
  constexpr int KS = L::KS, EPL = L::EPL, RING = L::RING, KCH = L::KCH;
  constexpr int KPS = STEP / KS;            // MFMA k-steps per pipeline step
  constexpr int MB = 32 * BMT;               // hidden rows per workgroup
  constexpr int HPAD = 16 / (int)sizeof(T);
  constexpr int HROW = KCH + HPAD;
  constexpr int EV = 16 / (int)sizeof(T);
  constexpr int HVEC = MB * KCH / EV / LM_THREADS;  // 16-byte vectors per thread per chunk
  __shared__ __attribute__((aligned(16))) T hs[2][MB][HROW];

  // XCD-aware tile order: dispatch id i runs on XCD i % 8; the nmb hidden-row blocks of one
  // vocabulary tile get ids that differ by multiples of 8.
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
  const int l32 = lane & 31, h2 = lane >> 5;
  const int m0 = mblk * MB;
  const int vbase = vtile * BV + wave * (VT_PER_WAVE * 32);

  // W row pointers of this lane (one per vocabulary tile); rows past V read nothing
  const T* wrow[VT_PER_WAVE];
  bool wok[VT_PER_WAVE];
#pragma unroll
  for (int vt = 0; vt < VT_PER_WAVE; ++vt) {
    const int v = vbase + vt * 32 + l32;
    wok[vt] = v < V;
    wrow[vt] = w + (size_t)(wok[vt] ? v : 0) * H;
  }

  frag ring[RING][VT_PER_WAVE][KPS];
  auto wload = [&](frag (&dst)[VT_PER_WAVE][KPS], int step) {
#pragma unroll
    for (int vt = 0; vt < VT_PER_WAVE; ++vt)
#pragma unroll
      for (int ks = 0; ks < KPS; ++ks) {
        const int h = step * STEP + ks * KS + EPL * h2;
        if (wok[vt]) {
          if constexpr (EPL == 8) dst[vt][ks] = *reinterpret_cast<const frag*>(wrow[vt] + h);
          else dst[vt][ks] = wrow[vt][h];
        } else {
          dst[vt][ks] = L::zero();
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
      hreg[i] = (m < M && h < H) ? *reinterpret_cast<const u32x4*>(hidden + (size_t)m * H + h)
                                 : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto hstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < HVEC; ++i) {
      const int v = tid + LM_THREADS * i;
      const int r = v / (KCH / EV), piece = v % (KCH / EV);
      *reinterpret_cast<u32x4*>(&hs[buf][r][piece * EV]) = hreg[i];
    }
  };

  f32x16 acc[BMT][VT_PER_WAVE];
#pragma unroll
  for (int mt = 0; mt < BMT; ++mt)
#pragma unroll
    for (int vt = 0; vt < VT_PER_WAVE; ++vt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mt][vt][j] = 0.f;

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
            const int hcol = sc * STEP + ks * KS + EPL * h2;
            if constexpr (EPL == 8) a = *reinterpret_cast<const frag*>(&hs[buf][mt * 32 + l32][hcol]);
            else a = hs[buf][mt * 32 + l32][hcol];
#pragma unroll
            for (int vt = 0; vt < VT_PER_WAVE; ++vt) acc[mt][vt] = L::mma(a, ring[r][vt][ks], acc[mt][vt]);
          }
        }
        if (s + RING < nsteps) wload(ring[r], s + RING);
        if (sc == SPC - 1 || s == nsteps - 1) {  // chunk boundary: publish the next hidden chunk
          if (chunk + 1 < nchunk) hstore(buf ^ 1);
          __syncthreads();
        }
      }
    }
  }

  // C[m][v]: lane l32 = vocabulary column, registers j = rows 8(j/4) + 4*h2 + j%4
#pragma unroll
  for (int mt = 0; mt < BMT; ++mt)
#pragma unroll
    for (int vt = 0; vt < VT_PER_WAVE; ++vt) {
      const int v = vbase + vt * 32 + l32;
      if (v >= V) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = m0 + mt * 32 + 8 * (j >> 2) + 4 * h2 + (j & 3);
        if (m < M) logits[(size_t)m * V + v] = acc[mt][vt][j];
      }
    }
}

template <typename T, int BMT>
int lm_launch(const void* hidden, const void* w, float* logits, int M, int H, int V, hipStream_t s) {
  const int nvt = (V + BV - 1) / BV;
  const int nmb = (M + 32 * BMT - 1) / (32 * BMT);
  unsigned grid;
  if (nmb == 1) grid = (unsigned)nvt;
  else grid = (unsigned)(((nvt + NXCD - 1) / NXCD) * NXCD * nmb);
  hipLaunchKernelGGL((lmhead_kernel<T, BMT>), dim3(grid), dim3(LM_THREADS), 0, s, (const T*)hidden,
                     (const T*)w, logits, M, H, V, nvt, nmb);
  return tt_launch_status();
}

}  // namespace

extern "C" int tt_lmhead_logits(const void* hidden, const void* w, float* logits, int M, int H,
                                int V, int dtype, void* stream) {
  if (!hidden || !w || !logits) return TT_ERR_ARG;
  if (M <= 0 || H <= 0 || V <= 0) return TT_ERR_ARG;
  if (dtype != TT_F32 && dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (H % 32 != 0) return TT_ERR_UNSUPPORTED;
  if ((uintptr_t)hidden % 16 || (uintptr_t)w % 16) return TT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == TT_BF16) {
    if (M <= 32) return lm_launch<bf16, 1>(hidden, w, logits, M, H, V, s);
    if (M <= 64) return lm_launch<bf16, 2>(hidden, w, logits, M, H, V, s);
    return lm_launch<bf16, 4>(hidden, w, logits, M, H, V, s);
  }
  if (M <= 32) return lm_launch<float, 1>(hidden, w, logits, M, H, V, s);
  return lm_launch<float, 4>(hidden, w, logits, M, H, V, s);
}
