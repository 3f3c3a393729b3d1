// Denoiser block attention ("Nemotron-Labs-TwoTower" wiki page, section "Architecture").
//
// A "unit" is one (sequence b, kv head g). Its key list is [k_ctx rows of b ; the S block rows],
// N_b = ctx_len[b] + S keys, and its query tile is the S*G rows (block position s, grouped head hh)
// that share kv head g (G = Hq/Hkv; the grouping is contiguous: query head h uses kv head h/G).
//
// Work split (flash-decoding with stream-K balance): the key lists of all units, laid end to end,
// form one key space of T keys; workgroup w takes keys [floor(w*T/W), floor((w+1)*T/W)). A range
// can span several units; each (workgroup, unit) piece either covers the whole unit (the output is
// normalised and written directly) or leaves an fp32 partial (unnormalised O, running max, sum)
// in slot w + u of the workspace, which attn_combine merges in a fixed order. Slot w + u is
// injective because walking the pieces in order raises w or u (or both) at every boundary.
//
// Inside a workgroup (8 waves, one 32-row query tile each): each K/V stage of KC keys is staged once in LDS and shared by all
// S*G query rows (up to 256), so every key byte is read from HBM once. Scores are computed
// transposed, S^T = K Q^T, on 32x32 MFMA tiles: the result layout gives each lane one query row
// (column lane%32) and 16 keys, so the row max and sum need one cross-half exchange only. The
// exponentials are written back into the same registers and used directly as the B operand of
// O^T = V^T P^T; the reduction order over keys inside a stage is a fixed permutation, applied to
// V when it is written transposed into LDS.
#include "common.h"

namespace {

constexpr int AT_THREADS = 512;
constexpr int AT_WAVES = AT_THREADS / TT_WAVE;
constexpr int KC = 64;          // keys per LDS stage
constexpr int QT = 32;          // query rows per MFMA tile
constexpr int MAX_ROWS = 256;   // S*G limit: 8 tiles, one per wave
constexpr int NT = MAX_ROWS / QT / AT_WAVES;
constexpr int AT_MAX_B = 1024;  // sequences handled by the in-workgroup prefix scan
constexpr float LOG2E = 1.4426950408889634f;

template <typename T>
struct Mf;

template <>
struct Mf<bf16> {
  static constexpr int KS = 16;   // reduction depth of v_mfma_f32_32x32x16_bf16
  static constexpr int EPL = 8;   // operand elements per lane
  static constexpr int VPAD = 8;  // Vt row padding (elements); keeps rows 16-byte aligned
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Position of key `k` (within a stage) in the transposed V rows. The score registers j=8u..8u+7
  // of lane half h hold keys 16u + 8(j%8/4) + 4h + j%4; MFMA u consumes them as reduction
  // indices 16u + 8h + j%8, so the position swaps key bits 2 and 3.
  __device__ static __forceinline__ int vpos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }
  __device__ static __forceinline__ frag pfrag(const f32x16& p, int u) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)p[8 * u + i];
    return f;
  }
};

template <>
struct Mf<float> {
  static constexpr int KS = 2;    // v_mfma_f32_32x32x2f32
  static constexpr int EPL = 1;
  static constexpr int VPAD = 1;  // odd row length: conflict-free column reads
  typedef float frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  // register j = u of lane half h holds key 8(u/4) + 4h + u%4 and feeds reduction index 2u + h
  __device__ static __forceinline__ int vpos(int k) {
    return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1);
  }
  __device__ static __forceinline__ frag pfrag(const f32x16& p, int u) { return p[u]; }
};

template <typename T, int D>
struct Smem {
  static constexpr int KPAD = 16 / (int)sizeof(T);
  static constexpr int KROW = D + KPAD;
  static constexpr int VROW = KC + Mf<T>::VPAD;
  T k[2][KC][KROW];
  T vt[2][D][VROW];
};

struct Scan {
  int pb[AT_MAX_B + 1];  // pb[b] = sum_{b' < b} (ctx_len[b'] + S)
  int tmp[AT_THREADS];
};

// Exclusive prefix sums of N_b = ctx_len[b] + S into sc.pb[0..B] (B <= AT_MAX_B).
__device__ void scan_lengths(Scan& sc, const int32_t* __restrict__ ctx_len, int B, int S) {
  const int t = threadIdx.x;
  constexpr int PER = AT_MAX_B / AT_THREADS;
  int v[PER];
  int loc = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    int b = t * PER + k;
    v[k] = (b < B) ? ctx_len[b] + S : 0;
    loc += v[k];
  }
  sc.tmp[t] = loc;
  __syncthreads();
  for (int off = 1; off < AT_THREADS; off <<= 1) {  // Hillis-Steele inclusive scan
    int x = (t >= off) ? sc.tmp[t - off] : 0;
    __syncthreads();
    sc.tmp[t] += x;
    __syncthreads();
  }
  int run = sc.tmp[t] - loc;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    sc.pb[t * PER + k] = run;
    run += v[k];
  }
  if (t == AT_THREADS - 1) sc.pb[AT_MAX_B] = run;
  __syncthreads();
}

// The workgroup whose key range holds global key x (ranges [floor(wT/W), floor((w+1)T/W))).
__device__ __forceinline__ int owner_of(int64_t x, int64_t T, int W) {
  return (int)(((x + 1) * W - 1) / T);
}

template <typename T, int D>
struct Args {
  const T* q;
  const T* kb;
  const T* vb;
  const T* kc;
  const T* vc;
  const int32_t* ctx_start;
  const int32_t* ctx_len;
  T* out;
  float* ws_o;   // [slots][R][D]
  float2* ws_ml; // [slots][R] (running max of raw scores, sum)
  int B, S, Hq, Hkv;
  int64_t ctx_rows;
  int W;
  float c;  // softmax_scale * log2(e)
};

template <typename T, int D>
__global__ __launch_bounds__(AT_THREADS, 1) void attn_partial(Args<T, D> A) {
  typedef Mf<T> MF;
  typedef typename MF::frag frag;
  constexpr int KS = MF::KS, EPL = MF::EPL;
  constexpr int EV = 16 / (int)sizeof(T);        // elements per 16-byte vector
  constexpr int NVR = D / EV;                    // vectors per key row
  constexpr int NVEC = KC * NVR / AT_THREADS;    // vectors per thread per stage (K, and V)
  static_assert(KC * NVR % AT_THREADS == 0, "stage split");

  __shared__ Smem<T, D> sm;
  __shared__ Scan sc;

  const int tid = threadIdx.x;
  const int lane = tid & (TT_WAVE - 1);
  const int wave = tid / TT_WAVE;
  const int l32 = lane & 31;
  const int hh2 = lane >> 5;  // lane half
  const int w = blockIdx.x;
  const int G = A.Hq / A.Hkv;
  const int R = A.S * G;
  const int U = A.B * A.Hkv;

  scan_lengths(sc, A.ctx_len, A.B, A.S);
  const int64_t Ttot = (int64_t)A.Hkv * sc.pb[A.B];
  const int64_t lo = (int64_t)w * Ttot / A.W;
  const int64_t hi = (int64_t)(w + 1) * Ttot / A.W;
  if (lo >= hi) return;

  // first unit whose key list ends after lo: binary search over sequences, then kv head
  int b;
  {
    int l = 0, r = A.B - 1;
    while (l < r) {  // largest b with Hkv*pb[b] <= lo
      int m = (l + r + 1) >> 1;
      if ((int64_t)A.Hkv * sc.pb[m] <= lo) l = m; else r = m - 1;
    }
    b = l;
  }
  int u = b * A.Hkv + (int)((lo - (int64_t)A.Hkv * sc.pb[b]) / (sc.pb[b + 1] - sc.pb[b]));

  for (; u < U; ++u) {
    const int bb = u / A.Hkv, g = u - bb * A.Hkv;
    const int N = sc.pb[bb + 1] - sc.pb[bb];
    const int64_t Ou = (int64_t)A.Hkv * sc.pb[bb] + (int64_t)g * N;
    if (Ou >= hi) break;
    const int ka = (int)max((int64_t)0, lo - Ou);
    const int ke = (int)min((int64_t)N, hi - Ou);
    const bool whole = (ka == 0 && ke == N);
    const int P = N - A.S;
    const int64_t cstart = A.ctx_start[bb];

    // ---- query fragments (B operand of S^T = K Q^T): lane holds row 32t + l32
    frag qf[NT][D / KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int tile = wave + AT_WAVES * nt;
      const int row = tile * QT + l32;
      const bool ok = row < R;
      const int s = ok ? row / G : 0, hq = ok ? g * G + row % G : 0;
      const T* qp = A.q + (((size_t)bb * A.S + s) * A.Hq + hq) * D;
#pragma unroll
      for (int ks = 0; ks < D / KS; ++ks) {
        if (ok) {
          if constexpr (EPL == 8) qf[nt][ks] = *reinterpret_cast<const frag*>(qp + KS * ks + EPL * hh2);
          else qf[nt][ks] = qp[KS * ks + hh2];
        } else {
          if constexpr (EPL == 8) { for (int i = 0; i < 8; ++i) qf[nt][ks][i] = (bf16)0.f; }
          else qf[nt][ks] = 0.f;
        }
      }
    }

    f32x16 o[NT][D / 32];
    float mrun[NT], lrun[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mrun[nt] = -INFINITY;
      lrun[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[nt][dt][j] = 0.f;
    }

    // ---- stage loader: global -> registers -> LDS
    u32x4 kreg[NVEC], vreg[NVEC];
    auto row_ptr = [&](const T* ctx, const T* blk, int key) -> const T* {
      return key < P ? ctx + ((size_t)g * A.ctx_rows + cstart + key) * D
                     : blk + (((size_t)bb * A.S + (key - P)) * A.Hkv + g) * D;
    };
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < NVEC; ++i) {
        const int v = tid + AT_THREADS * i;
        {  // K: consecutive threads walk a key row (coalesced rows)
          const int key = v / NVR, piece = v % NVR;
          const int kk = k0 + key;
          kreg[i] = (kk < ke) ? *reinterpret_cast<const u32x4*>(row_ptr(A.kc, A.kb, kk) + piece * EV)
                              : u32x4{0u, 0u, 0u, 0u};
        }
        {  // V: consecutive threads walk keys (conflict-free transposed LDS writes)
          const int key = v % KC, piece = v / KC;
          const int kk = k0 + key;
          vreg[i] = (kk < ke) ? *reinterpret_cast<const u32x4*>(row_ptr(A.vc, A.vb, kk) + piece * EV)
                              : u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto swrite = [&](int buf) {
#pragma unroll
      for (int i = 0; i < NVEC; ++i) {
        const int v = tid + AT_THREADS * i;
        {
          const int key = v / NVR, piece = v % NVR;
          *reinterpret_cast<u32x4*>(&sm.k[buf][key][piece * EV]) = kreg[i];
        }
        {
          const int key = v % KC, piece = v / KC;
          const int pos = MF::vpos(key);
          const T* e = reinterpret_cast<const T*>(&vreg[i]);
#pragma unroll
          for (int x = 0; x < EV; ++x) sm.vt[buf][piece * EV + x][pos] = e[x];
        }
      }
    };

    const int nst = (ke - ka + KC - 1) / KC;
    gload(ka);
    __syncthreads();  // previous piece's readers are done with both buffers
    swrite(0);
    __syncthreads();

    for (int st = 0; st < nst; ++st) {
      const int buf = st & 1;
      const int k0 = ka + st * KC;
      const int nvalid = min(KC, ke - k0);
      if (st + 1 < nst) gload(k0 + KC);

      // The stage is consumed as KC/32 sub-tiles of 32 keys, each a full online-softmax update,
      // which keeps only 32 keys of scores live per query tile.
#pragma unroll
      for (int kt = 0; kt < KC / 32; ++kt) {
        // ---- S^T tile: 32 keys on rows, query rows on columns
        f32x16 sacc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int j = 0; j < 16; ++j) sacc[nt][j] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / KS; ++ks) {
          frag a;
          if constexpr (EPL == 8) a = *reinterpret_cast<const frag*>(&sm.k[buf][kt * 32 + l32][KS * ks + EPL * hh2]);
          else a = sm.k[buf][kt * 32 + l32][KS * ks + hh2];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            if ((wave + AT_WAVES * nt) * QT < R) sacc[nt] = MF::mma(a, qf[nt][ks], sacc[nt]);
        }

        // ---- online softmax (base 2; raw-score max, scale folded into the exponent)
        const int kvalid = nvalid - kt * 32;  // keys of this sub-tile that exist
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if ((wave + AT_WAVES * nt) * QT >= R) continue;
          float mx = -INFINITY;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = 8 * (j >> 2) + 4 * hh2 + (j & 3);
            if (key >= kvalid) sacc[nt][j] = -INFINITY;
            mx = fmaxf(mx, sacc[nt][j]);
          }
          mx = fmaxf(mx, tt_shfl_xor(mx, 32));
          const float mnew = fmaxf(mrun[nt], mx);
          if (__ballot(mnew > mrun[nt])) {
            const float alpha = tt_exp2((mrun[nt] - mnew) * A.c);  // 0 on the first update
            lrun[nt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
              for (int j = 0; j < 16; ++j) o[nt][dt][j] *= alpha;
            mrun[nt] = mnew;
          }
          const float mc = mnew * A.c;
          float ls = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float p = tt_exp2(fmaf(sacc[nt][j], A.c, -mc));
            sacc[nt][j] = p;
            ls += p;
          }
          lrun[nt] += ls;
        }

        // ---- O^T += V^T P^T
        frag pf[NT][32 / KS];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int uu = 0; uu < 32 / KS; ++uu) pf[nt][uu] = MF::pfrag(sacc[nt], uu);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
          for (int uu = 0; uu < 32 / KS; ++uu) {
            frag a;
            if constexpr (EPL == 8) a = *reinterpret_cast<const frag*>(&sm.vt[buf][dt * 32 + l32][kt * 32 + KS * uu + EPL * hh2]);
            else a = sm.vt[buf][dt * 32 + l32][kt * 32 + KS * uu + hh2];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              if ((wave + AT_WAVES * nt) * QT < R) o[nt][dt] = MF::mma(a, pf[nt][uu], o[nt][dt]);
          }
        }
      }

      if (st + 1 < nst) swrite(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: direct normalised output, or an fp32 partial in slot w + u
    const size_t slot = (size_t)w + u;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int tile = wave + AT_WAVES * nt;
      if (tile * QT >= R) continue;
      const float ltot = lrun[nt] + tt_shfl_xor(lrun[nt], 32);
      const int row = tile * QT + l32;
      if (row >= R) continue;
      if (whole) {
        const int s = row / G, hq = g * G + row % G;
        T* op = A.out + (((size_t)bb * A.S + s) * A.Hq + hq) * D;
        const float inv = 1.f / ltot;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const int d = dt * 32 + 8 * jg + 4 * hh2;
            if constexpr (sizeof(T) == 2) {
              bf16x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[nt][dt][4 * jg + e] * inv);
              *reinterpret_cast<bf16x4*>(op + d) = v;
            } else {
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = o[nt][dt][4 * jg + e] * inv;
              *reinterpret_cast<f32x4*>(op + d) = v;
            }
          }
      } else {
        float* wp = A.ws_o + (slot * R + row) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const int d = dt * 32 + 8 * jg + 4 * hh2;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = o[nt][dt][4 * jg + e];
            *reinterpret_cast<f32x4*>(wp + d) = v;
          }
        if (hh2 == 0) A.ws_ml[slot * R + row] = make_float2(mrun[nt], ltot);
      }
    }
  }
}

// Merge the partials of units split across workgroups, in workgroup order (deterministic).
template <typename T, int D>
__global__ __launch_bounds__(AT_THREADS) void attn_combine(Args<T, D> A) {
  __shared__ Scan sc;
  constexpr int TPR = D / 4;              // threads per query row (4 values each)
  constexpr int RPB = AT_THREADS / TPR;   // rows per workgroup
  const int G = A.Hq / A.Hkv;
  const int R = A.S * G;
  const int u = blockIdx.y;
  const int bb = u / A.Hkv, g = u - bb * A.Hkv;
  scan_lengths(sc, A.ctx_len, A.B, A.S);
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int d = (threadIdx.x % TPR) * 4;
  if (row >= R) return;
  const int64_t Ttot = (int64_t)A.Hkv * sc.pb[A.B];
  const int N = sc.pb[bb + 1] - sc.pb[bb];
  const int64_t Ou = (int64_t)A.Hkv * sc.pb[bb] + (int64_t)g * N;
  const int wf = owner_of(Ou, Ttot, A.W), wl = owner_of(Ou + N - 1, Ttot, A.W);
  if (wf == wl) return;  // one workgroup held the whole unit and wrote the output itself
  float M = -INFINITY;
  for (int w = wf; w <= wl; ++w) M = fmaxf(M, A.ws_ml[((size_t)w + u) * R + row].x);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int w = wf; w <= wl; ++w) {
    const size_t slot = (size_t)w + u;
    const float2 ml = A.ws_ml[slot * R + row];
    const float sc_w = tt_exp2((ml.x - M) * A.c);
    L += ml.y * sc_w;
    const f32x4 v = *reinterpret_cast<const f32x4*>(A.ws_o + (slot * R + row) * D + d);
    acc += v * sc_w;
  }
  const float inv = 1.f / L;
  const int s = row / G, hq = g * G + row % G;
  T* op = A.out + (((size_t)bb * A.S + s) * A.Hq + hq) * D + d;
  if constexpr (sizeof(T) == 2) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x4*>(op) = v;
  } else {
    *reinterpret_cast<f32x4*>(op) = acc * inv;
  }
}

constexpr int MIN_KEYS_PER_WG = 128;
constexpr int AT_TARGET_WG = 256;

template <typename T, int D>
int launch(const void* q, const void* kb, const void* vb, const void* kc, const void* vc,
           const int32_t* cs, const int32_t* cl, void* out, int B, int S, int Hq, int Hkv,
           int64_t ctx_rows, int max_prefix, float scale, void* ws, size_t* ws_bytes,
           hipStream_t stream) {
  const int G = Hq / Hkv, R = S * G, U = B * Hkv;
  // One workgroup per compute unit of an MI355X-class gfx950 part (256 CUs), fewer when the key
  // space is small; a fixed count keeps the workspace size a pure function of the arguments.
  const int64_t tmax = (int64_t)U * ((int64_t)max_prefix + S);
  int W = (int)std::min<int64_t>((int64_t)AT_TARGET_WG, (tmax + MIN_KEYS_PER_WG - 1) / MIN_KEYS_PER_WG);
  if (W < 1) W = 1;
  const size_t slots = (size_t)W + U;
  const size_t o_bytes = tt_align_up(slots * R * D * sizeof(float), 256);
  const size_t need = o_bytes + tt_align_up(slots * R * sizeof(float2), 256);
  int st = tt_workspace_check(ws, ws_bytes, need);
  if (st != 0) return st < 0 ? st : TT_OK;
  if ((uintptr_t)ws % 256) return TT_ERR_ARG;
  Args<T, D> a;
  a.q = (const T*)q; a.kb = (const T*)kb; a.vb = (const T*)vb;
  a.kc = (const T*)kc; a.vc = (const T*)vc;
  a.ctx_start = cs; a.ctx_len = cl; a.out = (T*)out;
  a.ws_o = (float*)ws;
  a.ws_ml = (float2*)((char*)ws + o_bytes);
  a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.ctx_rows = ctx_rows; a.W = W;
  a.c = scale * LOG2E;
  hipLaunchKernelGGL((attn_partial<T, D>), dim3(W), dim3(AT_THREADS), 0, stream, a);
  if (tt_launch_status() != TT_OK) return TT_ERR_HIP;
  if (W > 1) {
    constexpr int RPB = AT_THREADS / (D / 4);
    hipLaunchKernelGGL((attn_combine<T, D>), dim3((R + RPB - 1) / RPB, U), dim3(AT_THREADS), 0,
                       stream, a);
    if (tt_launch_status() != TT_OK) return TT_ERR_HIP;
  }
  return TT_OK;
}

}  // namespace

extern "C" int tt_block_attn(const void* q, const void* k_blk, const void* v_blk, const void* k_ctx,
                             const void* v_ctx, const int32_t* ctx_start, const int32_t* ctx_len,
                             void* out, int B, int S, int Hq, int Hkv, int D, int64_t ctx_rows,
                             int max_prefix, float softmax_scale, int dtype, void* workspace,
                             size_t* workspace_bytes, void* stream) {
  if (!q || !k_blk || !v_blk || !ctx_start || !ctx_len || !out || !workspace_bytes) return TT_ERR_ARG;
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return TT_ERR_ARG;
  if (Hq % Hkv != 0 || ctx_rows < 0 || max_prefix < 0) return TT_ERR_ARG;
  if (max_prefix > 0 && (!k_ctx || !v_ctx)) return TT_ERR_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return TT_ERR_ARG;
  if (dtype != TT_F32 && dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return TT_ERR_UNSUPPORTED;
  if ((int64_t)S * (Hq / Hkv) > MAX_ROWS) return TT_ERR_UNSUPPORTED;
  if (B > AT_MAX_B) return TT_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * ((int64_t)max_prefix + S) >= ((int64_t)1 << 31)) return TT_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == TT_BF16) {
    if (D == 128) return launch<bf16, 128>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, ctx_rows, max_prefix, softmax_scale, workspace, workspace_bytes, s);
    return launch<bf16, 64>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, ctx_rows, max_prefix, softmax_scale, workspace, workspace_bytes, s);
  }
  if (D == 128) return launch<float, 128>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, ctx_rows, max_prefix, softmax_scale, workspace, workspace_bytes, s);
  return launch<float, 64>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, ctx_rows, max_prefix, softmax_scale, workspace, workspace_bytes, s);
}
