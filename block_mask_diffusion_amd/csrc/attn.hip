// Denoiser block attention ("Nemotron-Labs-TwoTower" wiki page, section "Architecture").
//
// A "unit" is one (sequence b, kv head g). Its key list is [k_ctx rows of b ; the S block rows],
// N_b = len_b + S keys (len_b = ctx_len[b] within the bounds of ctx_rows_of), and its query tile is the S*G rows (block position s, grouped head hh)
// that share kv head g (G = Hq/Hkv; the grouping is contiguous: query head h uses kv head h/G).
//
// Work split (flash-decoding with stream-K balance): the key lists of all units, laid end to end,
// form one key space of T keys; workgroup w takes keys [floor(w*T/W), floor((w+1)*T/W)). A range
// can span several units; each (workgroup, unit) piece either covers the whole unit (the output is
// normalised and written directly) or leaves an fp32 partial (O / l, with the running max m and
// the sum l) in slot w + u of the workspace, which attn_combine merges in
// a fixed order. Slot w + u is injective because walking the pieces in order raises w or u (or
// both) at every boundary.
//
// Inside a workgroup (8 waves, one 32-row query tile each): K/V stages of KC keys go straight from
// HBM into an LDS ring of NBUF stages (direct global->LDS loads) and are shared by all S*G query
// rows (up to 256), so every key byte is read from HBM once. Scores are computed transposed,
// S^T = K Q^T, on 32x32 MFMA tiles: the result layout gives each lane one query row (column
// lane%32) and 16 keys, so the row max and sum need one cross-half exchange only. The
// exponentials are written back into the same registers and used directly as the B operand of
// O^T = V^T P^T; the V^T operand is read from the row-major V stage with transposing LDS reads,
// in the key order of the score registers.
//
// The bf16 sub-tile loop is software-pipelined (a wave's softmax arithmetic runs between its own
// MFMAs) and unrolled over one turn of the ring, so that every LDS address is a register plus an
// immediate: with two waves per SIMD, each instruction a wave issues costs it an issue slot, and
// removing the per-sub-tile address and M0 arithmetic is what shortened the kernel (MI355X
// counters at 4 x 131072 keys: 22% fewer instructions, 13% fewer cycles). The schedule alone,
// without the unroll, did not change the time.
#include "common.h"

namespace {

constexpr int AT_THREADS = 512;
constexpr int AT_WAVES = AT_THREADS / TT_WAVE;
constexpr int QT = 32;          // query rows per MFMA tile, one tile per wave
constexpr int MAX_ROWS = 256;   // S*G limit: 8 tiles
constexpr int AT_MAX_B = 1024;  // sequences handled by the in-workgroup prefix scan
constexpr float LOG2E = 1.4426950408889634f;
static_assert(MAX_ROWS == QT * AT_WAVES, "8 query tiles per workgroup");
constexpr float RESCALE_LOG2 = 8.f;  // lazy-rescale threshold (log2 units)
// speculative probabilities (bf16 path): a lane's sum of its 16 above this takes the slow path
constexpr float RESCALE_SUM = 256.f;
// K/V stage loads: every key row is read exactly once, so they stream with the non-temporal
// policy
#ifndef TT_AT_DMA
#define TT_AT_DMA tt_dma16_nt
#endif

template <typename T>
struct Mf;

template <>
struct Mf<bf16> {
  static constexpr int KS = 16;   // reduction depth of v_mfma_f32_32x32x16_bf16
  static constexpr int EPL = 8;   // operand elements per lane
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // The P^T operand of MFMA u holds score registers 8u..8u+7, rounded to bf16. Register j of
  // lane half h holds key 8(j/4) + 4h + j%4 of the sub-tile, i.e. keys 16u + 4h + {0..3} and
  // 16u + 8 + 4h + {0..3}; the V^T operand is read in the same key order.
};

template <>
struct Mf<float> {
  static constexpr int KS = 2;    // v_mfma_f32_32x32x2f32
  static constexpr int EPL = 1;
  typedef float frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  // The P^T operand of MFMA u is score register u: key 8(u/4) + 4h + u%4 for lane half h,
  // reduction slot 2u + h.
};

// Stage geometry: KC keys per stage (64 for bf16, 32 for fp32), K and V stored row-major in an
// LDS ring of NBUF stages, written by direct global->LDS loads.
template <typename T>
constexpr int kc_of() { return sizeof(T) == 2 ? 64 : 32; }
constexpr int NBUF = 4;
constexpr int PD = 2;  // stages whose loads run ahead (two more are in use: K is read one
                       // sub-tile ahead of V)

template <typename T, int D>
struct Geo {
  static constexpr int KC = kc_of<T>();
  static constexpr int RB = D * (int)sizeof(T);        // bytes per key row
  static constexpr int GPR = RB / 16;                  // 16-byte granules per row
  static constexpr int RPC = 1024 / RB;                // rows per 1 KiB load chunk (64 lanes x 16 B)
  static constexpr int NCH = KC * RB / 1024;           // chunks per stage, for K and for V
  static constexpr int STAGE = KC * RB;                // bytes of K (or V) per stage
  static constexpr int DPW = 2 * NCH / AT_WAVES;       // load instructions per wave per stage
  static constexpr int RPW = RB >= 256 ? 1 : 256 / RB; // rows per 256-byte bank window
  static constexpr int GMASK = GPR - 1 < 15 ? GPR - 1 : 15;
  static_assert(NCH % AT_WAVES == 0, "chunks split over the waves");
  // XOR swizzle of the 16-byte granules of row r (an involution, applied on the load side):
  // K rows read 32 at a time at one logical granule -> spread over all banks;
  // V rows read 8 at a time by the transposing reads -> at most 2-way conflicts.
  __device__ static __forceinline__ int fk(int r) { return (r / RPW) & GMASK; }
  __device__ static __forceinline__ int fv(int r) {
    if constexpr (sizeof(T) == 2 && D == 128) return 4 * (r & 3);
    else if constexpr (sizeof(T) == 2 && D == 64) return 4 * ((r >> 1) & 1);
    else return fk(r);
  }
};

template <typename T, int D>
struct alignas(16) Ring {
  unsigned char k[NBUF][Geo<T, D>::STAGE];
  unsigned char v[NBUF][Geo<T, D>::STAGE];
};

template <int NT>
struct Scan {
  int pb[AT_MAX_B + 1];  // pb[b] = sum_{b' < b} (len_b' + S)
  int tmp[NT];
};

// The context rows [start, start + len) of sequence b that every kernel here uses: ctx_start[b]
// clamped to [0, ctx_rows], ctx_len[b] to [0, min(max_prefix, ctx_rows - start)]. Inside the
// caller's contract these are the values given. Outside it no access leaves k_ctx / v_ctx and the
// key-space sums stay within the bound the host checked (B Hkv (max_prefix + S) < 2^31).
struct CtxRows {
  int64_t start;
  int len;
};
__device__ __forceinline__ CtxRows ctx_rows_of(const int32_t* cs, const int32_t* cl, int b, int64_t ctx_rows,
                                               int max_prefix) {
  const int64_t st = min(max((int64_t)cs[b], (int64_t)0), ctx_rows);
  const int64_t cap = min((int64_t)max_prefix, ctx_rows - st);
  return CtxRows{st, (int)min(max((int64_t)cl[b], (int64_t)0), cap)};
}

// Exclusive prefix sums of N_b = len_b + S (len_b from ctx_rows_of) into sc.pb[0..B] (B <= AT_MAX_B), NT threads:
// thread t sums its PER consecutive lengths, a shuffle scan runs inside each wave, and the wave
// totals are added through LDS (two barriers).
template <int NT>
__device__ void scan_lengths(Scan<NT>& sc, const int32_t* __restrict__ ctx_start, const int32_t* __restrict__ ctx_len,
                             int B, int S, int64_t ctx_rows, int max_prefix) {
  const int t = threadIdx.x;
  constexpr int PER = AT_MAX_B / NT;
  constexpr int NW = NT / TT_WAVE;
  static_assert(NW <= TT_WAVE, "wave totals fit one wave");
  int v[PER];
  int loc = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    int b = t * PER + k;
    v[k] = (b < B) ? ctx_rows_of(ctx_start, ctx_len, b, ctx_rows, max_prefix).len + S : 0;
    loc += v[k];
  }
  const int lane = t & (TT_WAVE - 1), wv = t / TT_WAVE;
  int inc = loc;  // inclusive scan of loc inside the wave
#pragma unroll
  for (int off = 1; off < TT_WAVE; off <<= 1) {
    const int x = __shfl_up(inc, off, TT_WAVE);
    if (lane >= off) inc += x;
  }
  if (lane == TT_WAVE - 1) sc.tmp[wv] = inc;
  __syncthreads();
  int before = 0;  // totals of the waves before this one
  for (int k = 0; k < wv; ++k) before += sc.tmp[k];
  int run = before + inc - loc;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    sc.pb[t * PER + k] = run;
    run += v[k];
  }
  if (t == NT - 1) sc.pb[AT_MAX_B] = run;
  __syncthreads();
}

// The workgroup whose key range holds global key x (ranges [floor(wT/W), floor((w+1)T/W))).
__device__ __forceinline__ int owner_of(int64_t x, int64_t T, int W) {
  return (int)(((x + 1) * W - 1) / T);
}

// Element type of the split-K partial outputs (normalised O / l): fp32 for every input type. A
// bf16 partial would add a second rounding of up to 2^-8 |o| on top of the output's own bf16
// rounding, which for outputs near single value rows (|o| of a few units) breaks a 1e-2 bound.
template <typename T>
using PartT = float;

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
  // [slots][ceil(R/32)][D/8][2][32][4]: normalised partial output O / l in the MFMA output
  // layout of the wave that owns each 32-row tile (element (row, d) of a slot at
  // ((((row/32) D/8 + d/8) 2 + (d/4)%2) 32 + row%32) 4 + d%4). Each partial store instruction
  // then writes 1 KiB and each wave 32 contiguous KiB, spread over all memory channels; the
  // combine's read of one 4-element quad of consecutive rows is contiguous as well.
  PartT<T>* ws_o;
  float2* ws_ml;   // [slots][R]: (reference r of the partial in log2 units, i.e. a score times c;
                   // sum l of exp2(score c - r)); r = -inf for a partial with no visible key
  int B, S, Hq, Hkv;
  int64_t ctx_rows;
  int max_prefix;
  int W;
  float c;  // softmax_scale * log2(e)
};

#define LDS_PTR(T, p) TT_LDS_PTR(T, p)

// CAUSAL = false: the denoiser's block attention (bidirectional in the block).
// CAUSAL = true: the context tower's step over newly committed tokens: block row j is visible to
// block position s only for j <= s (the prefix is visible to every position).
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(AT_THREADS, 1) void attn_partial(Args<T, D> A) {
  typedef Mf<T> MF;
  typedef Geo<T, D> GE;
  typedef typename MF::frag frag;
  constexpr int KS = MF::KS, EPL = MF::EPL, KC = GE::KC, RB = GE::RB, GPR = GE::GPR;
  constexpr int SPS = KC / 32;                  // 32-key sub-tiles per stage
  constexpr int CPW = GE::NCH / AT_WAVES;       // K (and V) chunks per wave per stage
  constexpr int NQK = D / KS;                   // MFMAs of one sub-tile's scores
  constexpr int NDT = D / 32;                   // 32-wide d tiles of the output
  constexpr int NUU = 32 / KS;                  // MFMAs per d tile of one sub-tile's PV product
  constexpr int NPV = NDT * NUU;
  // bf16: software-pipelined sub-tile loop. fp32 (32 registers of operands per MFMA tile more)
  // runs the sub-tiles one after the other, which keeps it within the register file.
  constexpr bool PIPE = EPL == 8;

  __shared__ Ring<T, D> ring;
  __shared__ Scan<AT_THREADS> sc;

  const int tid = threadIdx.x;
  const int lane = tid & (TT_WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / TT_WAVE);  // uniform per wave
  const int l32 = lane & 31;
  const int hh2 = lane >> 5;  // lane half
  const int w = blockIdx.x;
  const int G = A.Hq / A.Hkv;
  const int R = A.S * G;
  const int U = A.B * A.Hkv;
  const bool active = wave * QT < R;  // this wave owns query rows [32 wave, 32 wave + 32)

  scan_lengths<AT_THREADS>(sc, A.ctx_start, A.ctx_len, A.B, A.S, A.ctx_rows, A.max_prefix);
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

  // Per-lane byte offsets that are the same for every piece, stage and sub-tile (bf16 path): the
  // K and V^T fragment reads inside a stage slot (the slot and the sub-tile add constants, since
  // the swizzles repeat every 16 rows and sub-tiles are 32 rows apart), and the stage loads'
  // sources relative to the stage's first key row.
  static_assert(!PIPE || (32 % (GE::RPW * (GE::GMASK + 1)) == 0), "K swizzle repeats within 32 rows");
  typedef __attribute__((address_space(3))) const unsigned char* lds_cptr;
  lds_cptr koff[NQK], voff[NDT];
  uint32_t dkoff[CPW], dvoff[CPW];
  uint32_t lds_k0 = 0;  // LDS address of this wave's first load chunk in stage slot 0 (K)
  if constexpr (PIPE) {
    const unsigned char* rk = &ring.k[0][0];
    const unsigned char* rv = &ring.v[0][0];
#pragma unroll
    for (int ks = 0; ks < NQK; ++ks)
      koff[ks] = TT_LDS_PTR(const unsigned char, rk + l32 * RB + 16 * ((2 * ks + hh2) ^ GE::fk(l32)));
    const int G4 = lane >> 4, jj = lane & 15;
    const int r0 = 4 * (G4 >> 1) + (jj >> 2);  // + 32 kt + 16 uu + 8 rd: same V swizzle
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = dt * 32 + 16 * (G4 & 1) + 4 * (jj & 3);
      voff[dt] = TT_LDS_PTR(const unsigned char, rv + r0 * RB + 16 * ((d >> 3) ^ GE::fv(r0)) + 2 * (d & 7));
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int r = (wave * CPW + c) * GE::RPC + lane / GPR, slot = lane % GPR;
      dkoff[c] = r * RB + 16 * (slot ^ GE::fk(r));
      dvoff[c] = r * RB + 16 * (slot ^ GE::fv(r));
    }
    lds_k0 = tt_lds_addr(&ring.k[0][wave * CPW * 1024]);
  }

  for (; u < U; ++u) {
    const int bb = u / A.Hkv, g = u - bb * A.Hkv;
    const int N = sc.pb[bb + 1] - sc.pb[bb];
    const int64_t Ou = (int64_t)A.Hkv * sc.pb[bb] + (int64_t)g * N;
    if (Ou >= hi) break;
    const int ka = (int)max((int64_t)0, lo - Ou);
    const int ke = (int)min((int64_t)N, hi - Ou);
    const bool whole = (ka == 0 && ke == N);
    const int P = N - A.S;
    const int64_t cst = ctx_rows_of(A.ctx_start, A.ctx_len, bb, A.ctx_rows, A.max_prefix).start;
    const T* kctx = A.kc + ((size_t)g * A.ctx_rows + cst) * D;  // row 0 of this unit
    const T* vctx = A.vc + ((size_t)g * A.ctx_rows + cst) * D;
    const size_t blk_stride = (size_t)A.Hkv * D;                             // between block rows
    const T* kblk = A.kb + ((size_t)bb * A.S * A.Hkv + g) * D;
    const T* vblk = A.vb + ((size_t)bb * A.S * A.Hkv + g) * D;

    // ---- query fragments (B operand of S^T = K Q^T): lane holds query row `row` of the unit
    const int row = wave * QT + l32;
    const bool row_ok = active && row < R;
    frag qf[NQK];
    {
      const int s = row_ok ? row / G : 0, hq = row_ok ? g * G + row % G : 0;
      const T* qp = A.q + (((size_t)bb * A.S + s) * A.Hq + hq) * D;
#pragma unroll
      for (int ks = 0; ks < NQK; ++ks) {
        if (row_ok) {
          if constexpr (EPL == 8) qf[ks] = *reinterpret_cast<const frag*>(qp + KS * ks + EPL * hh2);
          else qf[ks] = qp[KS * ks + hh2];
        } else {
          if constexpr (EPL == 8) { for (int i = 0; i < 8; ++i) qf[ks][i] = (bf16)0.f; }
          else qf[ks] = 0.f;
        }
      }
      // Wait for the query loads here, on every path, with a wait the compiler sees: otherwise
      // its wait-count pass may place a full vmcnt(0) wait inside the sub-tile loop (it does not
      // see the stage loads, which are inline asm), and that would drain the stage prefetch.
      __builtin_amdgcn_s_waitcnt(TT_WAIT_VMCNT0);
    }

    f32x16 o[NDT];
    float mrun = -INFINITY, lrun = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;

    // ---- stage loads: global -> LDS directly
    const int nkeys = ke - ka;
    // Per-lane load sources of this piece. Chunk c of a stage holds rows [c*RPC, c*RPC+RPC); lane i
    // writes LDS bytes [16i, 16i+16) of the chunk = granule slot i%GPR of row i/GPR, which holds
    // logical granule slot ^ f(row); the row and so the swizzle are the same in every stage.
    // Fast path (uniform per stage): all KC keys of the stage are context keys of this piece, so
    // each source is the piece's first stage address plus st * KC rows. Otherwise each key is
    // clamped to the piece and taken from the context or the block rows; keys past the piece end
    // re-read its last key (their scores are masked and their probabilities are exactly 0).
    const unsigned char* kfast[CPW];
    const unsigned char* vfast[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int r = (wave * CPW + c) * GE::RPC + lane / GPR, slot = lane % GPR;
      kfast[c] = reinterpret_cast<const unsigned char*>(kctx + (size_t)(ka + r) * D) + 16 * (slot ^ GE::fk(r));
      vfast[c] = reinterpret_cast<const unsigned char*>(vctx + (size_t)(ka + r) * D) + 16 * (slot ^ GE::fv(r));
    }
    const int fast_end = min(P, ke);  // keys below this are context keys of the piece
    // one load of stage st: chunk c of K (kv = 0) or of V (kv = 1)
    auto issue_chunk = [&](int st, int c, int kv) {
      const int buf = st % NBUF;
      const int k0 = ka + st * KC;
      const int chunk = wave * CPW + c;
      unsigned char* dst = kv ? &ring.v[buf][chunk * 1024] : &ring.k[buf][chunk * 1024];
      if (k0 + KC <= fast_end) {
        TT_AT_DMA((kv ? vfast[c] : kfast[c]) + (size_t)st * KC * RB, tt_lds_addr(dst));
        return;
      }
      const int r = chunk * GE::RPC + lane / GPR, slot = lane % GPR;
      int key = k0 + r;
      key = key < ke ? key : ke - 1;
      const int g = slot ^ (kv ? GE::fv(r) : GE::fk(r));
      const T* src = kv ? (key < P ? vctx + (size_t)key * D : vblk + (size_t)(key - P) * blk_stride)
                        : (key < P ? kctx + (size_t)key * D : kblk + (size_t)(key - P) * blk_stride);
      TT_AT_DMA(reinterpret_cast<const unsigned char*>(src) + 16 * g, tt_lds_addr(dst));
    };
    auto issue_stage = [&](int st) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        issue_chunk(st, c, 0);
        issue_chunk(st, c, 1);
      }
    };
    // stage st resident: wait for this wave's loads of stage st (the later stages stay in flight),
    // then a barrier so every wave's loads of stage st are in LDS
    auto stage_ready = [&](int st, int nst) {
      const int later = min(nst - 1, st + PD - 1) - st;  // stages issued after st
      if (later >= 2) tt_wait_vmem<2 * GE::DPW>();
      else if (later == 1) tt_wait_vmem<GE::DPW>();
      else tt_wait_vmem<0>();
      tt_lds_barrier();
    };

    // K fragments (A operand of S^T = K Q^T) of sub-tile kt of a stage: lane holds key 32kt + l32
    auto kread = [&](const unsigned char* kb_, int kt, frag (&kf)[NQK]) {
      const int r = kt * 32 + l32;
      const unsigned char* rp = kb_ + r * RB;
      const int f = GE::fk(r);
#pragma unroll
      for (int ks = 0; ks < NQK; ++ks) {
        if constexpr (EPL == 8) {
          kf[ks] = *reinterpret_cast<const frag*>(rp + 16 * ((2 * ks + hh2) ^ f));
        } else {
          const int d = KS * ks + hh2;
          kf[ks] = *reinterpret_cast<const float*>(rp + 16 * ((d >> 2) ^ f) + 4 * (d & 3));
        }
      }
    };
    // V^T fragment of MFMA uu / d-tile dt: keys of the P registers 8uu..8uu+7 of this lane half
    auto vfrag = [&](const unsigned char* vb_, int kt, int uu, int dt) -> frag {
      if constexpr (EPL == 8) {
        // two transposing reads: 16-lane group G, lane j of it gets V[kb + e][d0 + j], e = 0..3,
        // when source lane j points at V[kb + j/4][d0 + 4*(j%4)]
        const int G4 = lane >> 4, j = lane & 15;
        const int d = dt * 32 + 16 * (G4 & 1) + 4 * (j & 3);
        frag f;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const int r = kt * 32 + 16 * uu + 4 * (G4 >> 1) + 8 * rd + (j >> 2);
          const unsigned char* p = vb_ + r * RB + 16 * ((d >> 3) ^ GE::fv(r)) + 2 * (d & 7);
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p));
          bf16x4 y = __builtin_bit_cast(bf16x4, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) f[4 * rd + e] = y[e];
        }
        return f;
      } else {
        // fp32: register uu of lane half h holds key 8(uu/4) + 4h + uu%4
        const int r = kt * 32 + 8 * (uu >> 2) + 4 * hh2 + (uu & 3);
        const int d = dt * 32 + l32;
        return *reinterpret_cast<const float*>(vb_ + r * RB + 16 * ((d >> 2) ^ GE::fv(r)) + 4 * (d & 3));
      }
    };

    // The pending PV product: V^T fragments and probabilities of the previous sub-tile. They start
    // at zero, so the first sub-tile's "previous" product adds nothing.
    frag va[NDT][NUU];
    frag pf[NUU];
#pragma unroll
    for (int uu = 0; uu < NUU; ++uu) {
      if constexpr (EPL == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[uu][i] = (bf16)0.f;
      } else {
        pf[uu] = 0.f;
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) va[dt][uu] = pf[uu];
    }
    // MFMA i of the pending PV product; consecutive ones go to different accumulators
    auto pv_mma = [&](auto i) {
      constexpr int I = decltype(i)::value, dt = I % NDT, uu = I / NDT;
      o[dt] = MF::mma(va[dt][uu], pf[uu], o[dt]);
    };
    // MFMA i of the scores of one sub-tile (one chain, from zero)
    auto qk_mma = [&](const frag (&kf)[NQK], f32x16& acc, auto i) {
      constexpr int I = decltype(i)::value;
      if constexpr (I == 0) {
        f32x16 z;
#pragma unroll
        for (int j = 0; j < 16; ++j) z[j] = 0.f;
        acc = MF::mma(kf[0], qf[0], z);
      } else {
        acc = MF::mma(kf[I], qf[I], acc);
      }
    };
    // Score register j of lane half h holds key 8(j/4) + 4h + j%4 of the sub-tile. Keys past the
    // piece end, and (causal) block rows after the query's own block position, get -inf.
    const int h4 = 4 * hh2;
    auto mask = [&](f32x16& s, int kvalid, int kfirst) {
      const int climit = (CAUSAL ? row / G + P - kfirst : 0);  // causal: keys above it are hidden
      int h4o = h4;
      asm volatile("" : "+v"(h4o));  // opaque here: the 16 key indices are not kept across steps
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = 8 * (j >> 2) + (j & 3);
        if (h4o + c >= kvalid) s[j] = -INFINITY;
        if constexpr (CAUSAL) {
          if (h4o + c > climit) s[j] = -INFINITY;
        }
      }
    };

    const int nsub = (nkeys + 31) / 32;
    const int nst = (nkeys + KC - 1) / KC;
    tt_wait_vmem<0>();   // the previous piece's partial stores; the load counting below starts clean
    __syncthreads();     // previous piece's readers are done with the ring
#pragma unroll
    for (int st = 0; st < PD; ++st)
      if (st < nst) issue_stage(st);
    stage_ready(0, nst);
    if (PD < nst) issue_stage(PD);

    // Row max of sub-tile j (after its masking), with the pending PV MFMAs issued between its
    // steps when with_pv is set; then the lazy rescale. Returns the sub-tile's exponent offset.
    auto row_max = [&](f32x16& sc, int j, auto with_pv) -> float {
      const int kvalid = nkeys - 32 * j;
      const int kfirst = ka + 32 * j;  // index in the unit's key list of the sub-tile's first key
      if (kvalid < 32 || (CAUSAL && kfirst + 32 > P)) mask(sc, kvalid, kfirst);
      float mx = -INFINITY;
      auto vmax = [&](auto e) { mx = fmaxf(mx, sc[decltype(e)::value]); };
      if constexpr (decltype(with_pv)::value) tt_interleave<NPV, 16, 0>(pv_mma, vmax, [](auto) {});
      else tt_static_for<16>(vmax);
      mx = tt_max_halves(mx);
      // Lazy rescale: the reference max only moves when a row's max grows by more than
      // 2^8 in the exponent; exponentials stay <= 256 and the final normalisation is exact.
      if (__ballot((mx - mrun) * A.c > RESCALE_LOG2)) {
        const float mnew = fmaxf(mrun, mx);
        // 0 on the first update; 1 for a row that has seen no visible key yet (causal), where
        // both maxima are -inf and their difference would be NaN
        const float alpha = (CAUSAL && mnew == -INFINITY) ? 1.f : tt_exp2((mrun - mnew) * A.c);
        lrun *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int q = 0; q < 16; ++q) o[dt][q] *= alpha;
        mrun = mnew;
      }
      // (causal: a row may have no visible key yet in this piece; its probabilities are 0)
      return (CAUSAL && mrun == -INFINITY) ? 0.f : mrun * A.c;
    };
    // Exponentials of a sub-tile (scores sc, exponent offset mc) into the P^T operand and the row
    // sum, with its V^T reads (vld(l): fragment l) and, when with_qk is set, the score MFMAs of the
    // next sub-tile (K fragments kf, into sn) issued between their steps.
    auto expo = [&](f32x16& sc, float mc, auto with_qk, const frag (&kf)[NQK], f32x16& sn, auto&& vld) {
      float ps = 0.f;  // fp32: the sub-tile's row sum, added to lrun at the end
      // each pair of bf16 probabilities goes to the row sum exactly as the PV product uses it
      auto vexp = [&](auto e) {
        constexpr int E = decltype(e)::value;
        sc[E] = tt_exp2(fmaf(sc[E], A.c, -mc));
        if constexpr (EPL == 8) {
          if constexpr (E % 2 == 1) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 one = {(bf16)1.f, (bf16)1.f};
            bf16x2 pr;
            pr[0] = (bf16)sc[E - 1];
            pr[1] = (bf16)sc[E];
            pf[E / 8][E % 8 - 1] = pr[0];
            pf[E / 8][E % 8] = pr[1];
            lrun = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lrun, false);
          }
        } else {
          pf[E] = sc[E];  // fp32: score register E is the P^T operand of MFMA E
          ps += sc[E];
        }
      };
      if constexpr (decltype(with_qk)::value) {
        tt_interleave<NQK, 16, NPV>([&](auto i) { qk_mma(kf, sn, i); }, vexp, vld);
      } else {
        tt_static_for<16>(vexp);
        tt_static_for<NPV>(vld);
      }
      if constexpr (EPL != 8) lrun += ps;
    };

    f32x16 sa, sb;
    float mc_final = 0.f;  // bf16 path: the reference its partial is relative to (log2 units)
    if constexpr (PIPE) {
      // Stage loads of the bf16 path with compile-time ring slot BUF: fast stages from the
      // piece's context rows through one scalar base per stage, others through issue_chunk.
      const unsigned char* kpiece = tt_uniform(reinterpret_cast<const unsigned char*>(kctx) + (size_t)ka * RB);
      const unsigned char* vpiece = tt_uniform(reinterpret_cast<const unsigned char*>(vctx) + (size_t)ka * RB);
      auto issue_stage_c = [&](auto buf, int st) {
        constexpr int BUF = decltype(buf)::value;
        if (ka + st * KC + KC <= fast_end) {
          const unsigned char* sk = kpiece + (size_t)st * KC * RB;
          const unsigned char* sv = vpiece + (size_t)st * KC * RB;
          if constexpr (CPW == 2) {  // head_dim 128: two K and two V chunks, one asm block
            tt_dma16x4_snt<BUF * GE::STAGE, BUF * GE::STAGE + 1024, (NBUF + BUF) * GE::STAGE,
                           (NBUF + BUF) * GE::STAGE + 1024>(dkoff[0], dkoff[1], dvoff[0], dvoff[1], sk,
                                                             sv, lds_k0);
          } else {
            tt_static_for<CPW>([&](auto c) {
              constexpr int C = decltype(c)::value;
              tt_dma16_snt<BUF * GE::STAGE + C * 1024>(dkoff[C], sk, lds_k0);
              tt_dma16_snt<(NBUF + BUF) * GE::STAGE + C * 1024>(dvoff[C], sv, lds_k0);
            });
          }
        } else {
          issue_stage(st);
        }
      };
      // K fragments of sub-tile KT of ring slot BUF
      auto kread_c = [&](auto buf, auto kt, frag (&kf)[NQK]) {
        constexpr int OFF = decltype(buf)::value * GE::STAGE + decltype(kt)::value * 32 * RB;
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks)
          kf[ks] = *reinterpret_cast<__attribute__((address_space(3))) const frag*>(koff[ks] + OFF);
      };
      // V^T fragment l (d tile l % NDT, MFMA l / NDT) of sub-tile KT of ring slot BUF: two
      // transposing reads (see vfrag)
      auto vread_c = [&](auto buf, auto kt, auto l) {
        constexpr int L = decltype(l)::value, dt = L % NDT, uu = L / NDT;
        constexpr int OFF = decltype(buf)::value * GE::STAGE + (decltype(kt)::value * 32 + 16 * uu) * RB;
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        frag f;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<__attribute__((address_space(3))) s16x4*>(
                  const_cast<__attribute__((address_space(3))) unsigned char*>(voff[dt] + OFF + 8 * rd * RB)));
          bf16x4 y = __builtin_bit_cast(bf16x4, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) f[4 * rd + e] = y[e];
        }
        va[dt][uu] = f;
      };

      // Software pipeline over the piece's 32-key sub-tiles. Step j holds the scores of sub-tile
      // j (sc) and the pending PV product of sub-tile j - 1; it reads the K fragments of sub-tile
      // j + 1 (after the barrier that makes its stage resident), issues the PV MFMAs of sub-tile
      // j - 1, then the score MFMAs of sub-tile j + 1 (into sn) with the probabilities and the
      // V^T reads of sub-tile j between them.
      // The probabilities are speculative: they are taken against the row's current reference
      // (the max of the piece's first sub-tile, raised when needed) without waiting for the
      // sub-tile's own row max. When this lane's sum of them passes 2^8 (some score rose about 8
      // log2 units above the reference), the sub-tile takes a slow path that moves the reference
      // to the row max, rescales O and l, and recomputes its probabilities from its scores, which
      // stay in registers until the check. On ordinary inputs no row max is taken in the loop.
      // The last step's score MFMAs read a stale ring slot; those scores are never used. K is
      // read one sub-tile ahead of V, so at a barrier two stages are in use. The loop runs NPH
      // steps per iteration (one turn of the ring), so ring slots and sub-tile offsets are
      // compile-time constants and every LDS address is a register plus an immediate.
      constexpr int NPH = NBUF * SPS;
      float mc = 0.f;  // the reference, in log2 units (a score times c)
      // probabilities of score registers 4Q..4Q+3 against mc, rounded to bf16 into the P^T
      // operand and added (as rounded) to ps[Q % 2]: four exponent arguments, four exponentials,
      // then the packing, so that no result is used right after the instruction that makes it
      auto pexp4 = [&](const f32x16& sc, float (&ps)[2], int q) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(bf16)1.f, (bf16)1.f};
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = fmaf(sc[4 * q + i], A.c, -mc);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = tt_exp2(x[i]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x2 pr;
          pr[0] = (bf16)x[2 * h];
          pr[1] = (bf16)x[2 * h + 1];
          if constexpr (EPL == 8) {
            pf[q / 2][4 * (q % 2) + 2 * h] = pr[0];
            pf[q / 2][4 * (q % 2) + 2 * h + 1] = pr[1];
          }
          ps[q % 2] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, ps[q % 2], false);
        }
      };
      auto mask_at = [&](f32x16& sc, int j) {
        const int kvalid = nkeys - 32 * j;
        const int kfirst = ka + 32 * j;  // index in the unit's key list of the sub-tile's first key
        if (kvalid < 32 || (CAUSAL && kfirst + 32 > P)) mask(sc, kvalid, kfirst);
      };
      auto rowmax = [&](const f32x16& sc) {
        float mx = sc[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
        return tt_max_halves(mx);
      };
      if (active) {
        // prologue: the scores of sub-tile 0 and, from their row max, the row's first reference
        // (-inf: no key of the piece is visible to the row, its probabilities are all 0)
        frag kf[NQK];
        kread_c(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, kf);
        tt_static_for<NQK>([&](auto i) { qk_mma(kf, sa, i); });
        mask_at(sa, 0);
        const float mx = rowmax(sa);
        mc = (mx == -INFINITY) ? 0.f : mx * A.c;
      }
      auto step = [&](auto ph, auto act, int j, f32x16& sc, f32x16& sn) {
        constexpr int PH = decltype(ph)::value, PN = PH + 1;
        constexpr int BUF = (PH / SPS) % NBUF, KT = PH % SPS;
        constexpr int BUFN = (PN / SPS) % NBUF, KTN = PN % SPS;
        const int jn = j + 1;
        if constexpr (KTN == 0) {
          if (jn < nsub) {  // sub-tile j + 1 opens a stage: make it resident
            const int stn = jn / SPS;
            stage_ready(stn, nst);  // every wave is done with stage stn - 2
            if (stn + PD < nst) issue_stage_c(std::integral_constant<int, (BUFN + PD) % NBUF>{}, stn + PD);
          }
        }
        if constexpr (!decltype(act)::value) return;  // a wave without query rows: loads only
        frag kf[NQK];
        kread_c(std::integral_constant<int, BUFN>{}, std::integral_constant<int, KTN>{}, kf);
        if (j > 0) mask_at(sc, j);
        tt_static_for<NPV>(pv_mma);
        float ps[2] = {0.f, 0.f};
        tt_interleave<NQK, 4, NPV>([&](auto i) { qk_mma(kf, sn, i); },
                                   [&](auto q) { pexp4(sc, ps, decltype(q)::value); },
                                   [&](auto l) {
                                     vread_c(std::integral_constant<int, BUF>{}, std::integral_constant<int, KT>{}, l);
                                   });
        // speculation check (see above); the PV MFMAs of j - 1 have all been issued, so O can be
        // rescaled here before the PV product of j adds to it
        if (__builtin_expect(__ballot(ps[0] + ps[1] > RESCALE_SUM) != 0, 0)) {
          const float mcn = fmaxf(mc, rowmax(sc) * A.c);
          const float alpha = tt_exp2(mc - mcn);
          lrun *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int q = 0; q < 16; ++q) o[dt][q] *= alpha;
          mc = mcn;
          ps[0] = ps[1] = 0.f;
          tt_static_for<4>([&](auto q) { pexp4(sc, ps, decltype(q)::value); });
        }
        lrun += ps[0] + ps[1];
      };
      auto run = [&](auto act) {
        for (int j0 = 0; j0 < nsub; j0 += NPH) {
          tt_static_for<NPH>([&](auto ph) {
            constexpr int PH = decltype(ph)::value;
            if (j0 + PH < nsub) {
              if constexpr (PH % 2 == 0) step(ph, act, j0 + PH, sa, sb);
              else step(ph, act, j0 + PH, sb, sa);
            }
          });
        }
      };
      if (active) run(std::true_type{});
      else run(std::false_type{});
      if (active) tt_static_for<NPV>(pv_mma);  // the last sub-tile's PV product
      mc_final = mc;
    } else {
      // One sub-tile after the other: scores, softmax, PV product.
      for (int j = 0; j < nsub; ++j) {
        if (j > 0 && j % SPS == 0) {
          stage_ready(j / SPS, nst);
          if (j / SPS + PD < nst) issue_stage(j / SPS + PD);
        }
        if (!active) continue;
        frag kf[NQK];
        kread(ring.k[(j / SPS) % NBUF], j % SPS, kf);
        tt_static_for<NQK>([&](auto i) { qk_mma(kf, sa, i); });
        const float mc = row_max(sa, j, std::false_type{});
        const unsigned char* vst = ring.v[(j / SPS) % NBUF];
        const int kt = j % SPS;
        expo(sa, mc, std::false_type{}, kf, sb, [&](auto l) {
          constexpr int L = decltype(l)::value, dt = L % NDT, uu = L / NDT;
          va[dt][uu] = vfrag(vst, kt, uu, dt);
        });
        tt_static_for<NPV>(pv_mma);
      }
    }

    // ---- epilogue: direct normalised output, or a normalised partial in slot w + u
    if (active) {
      const size_t slot = (size_t)w + u;
      const float ltot = lrun + tt_shfl_xor(lrun, 32);
      if (row < R) {
        if (whole) {
          const int s = row / G, hq = g * G + row % G;
          T* op = A.out + (((size_t)bb * A.S + s) * A.Hq + hq) * D;
          const float inv = 1.f / ltot;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
              const int d = dt * 32 + 8 * jg + 4 * hh2;
              if constexpr (sizeof(T) == 2) {
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[dt][4 * jg + e] * inv);
                *reinterpret_cast<bf16x4*>(op + d) = v;
              } else {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * jg + e] * inv;
                *reinterpret_cast<f32x4*>(op + d) = v;
              }
            }
        } else {
          typedef PartT<T> PT;
          typedef PT pvec __attribute__((ext_vector_type(4)));
          PT* wp = A.ws_o + ((slot * ((R + 31) / 32) + wave) * (D / 8) * 64 + lane) * 4;
          // (causal: a row with no visible key in this piece leaves an empty partial)
          const float inv = (CAUSAL && ltot == 0.f) ? 0.f : 1.f / ltot;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
              pvec v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = (PT)(o[dt][4 * jg + e] * inv);
              *reinterpret_cast<pvec*>(wp + (dt * 4 + jg) * 256) = v;
            }
          const float ref = PIPE ? mc_final : mrun * A.c;
          if (hh2 == 0) A.ws_ml[slot * R + row] = make_float2(ltot == 0.f ? -INFINITY : ref, ltot);
        }
      }
    }
  }
}

constexpr int CB_THREADS = 128;

// Block-wide sum of two 64-bit values (CB_THREADS threads).
__device__ __forceinline__ void block_sum2(int64_t& a, int64_t& b) {
  __shared__ int64_t red[2][CB_THREADS / TT_WAVE];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off, TT_WAVE);
    b += __shfl_xor(b, off, TT_WAVE);
  }
  const int wv = threadIdx.x / TT_WAVE;
  if ((threadIdx.x & (TT_WAVE - 1)) == 0) {
    red[0][wv] = a;
    red[1][wv] = b;
  }
  __syncthreads();
  a = 0;
  b = 0;
#pragma unroll
  for (int k = 0; k < CB_THREADS / TT_WAVE; ++k) {
    a += red[0][k];
    b += red[1][k];
  }
}

// Split-K merge of a unit's normalised partials (references r_k in log2 units, R their max):
// O = sum_k 2^(r_k - R) l_k Ohat_k / sum_k 2^(r_k - R) l_k. Workgroup = CB_RB query rows x QB quads (4 consecutive output elements)
// of one unit, rows fastest, so the 16-byte partial loads of consecutive threads are contiguous; thread (row rr, quad qq, group sg) owns one quad of its row and the
// partials of workgroups wf + sg, wf + sg + NSG, ... (CB loads in flight together); the NSG
// groups of a row are merged in the order sg = 0, 1, ... through LDS, a fixed order, so the
// result is reproducible. Many partials per unit (long sequences) use several groups per quad.
constexpr int CB_RB = 16;
template <typename T, int D, int NSG>
__global__ __launch_bounds__(CB_THREADS) void attn_combine(Args<T, D> A) {
  typedef PartT<T> PT;
  constexpr int VPT = 16 / (int)sizeof(PT);  // elements per thread (one 16-byte load)
  static_assert(VPT == 4, "fp32 partials, read one 4-element quad per thread");
  constexpr int NQ = D / VPT;                // quads per row
  constexpr int QB = CB_THREADS / (CB_RB * NSG);  // quads per workgroup
  static_assert(QB >= 1 && QB * CB_RB * NSG == CB_THREADS && NQ % QB == 0, "combine geometry");
  constexpr int CB = 8;                      // partials per group whose loads are in flight together
  const int G = A.Hq / A.Hkv;
  const int R = A.S * G;
  const int u = blockIdx.x;    // unit on x (up to B * Hkv workgroups), row block on y, quads on z
  const int rr = threadIdx.x % CB_RB;
  const int qq = (threadIdx.x / CB_RB) % QB;
  const int sg = threadIdx.x / (CB_RB * QB);
  const int row = blockIdx.y * CB_RB + rr;
  const int quad = blockIdx.z * QB + qq;
  const int RW = (R + 31) / 32;  // 32-row tiles of the partials
  const int bb = u / A.Hkv, g = u - bb * A.Hkv;
  // key-space offsets: sum of N_b' = len_b' + S over b' < bb, and over all b'
  int64_t before = 0, total = 0;
  for (int b2 = threadIdx.x; b2 < A.B; b2 += CB_THREADS) {
    const int64_t n = (int64_t)ctx_rows_of(A.ctx_start, A.ctx_len, b2, A.ctx_rows, A.max_prefix).len + A.S;
    total += n;
    if (b2 < bb) before += n;
  }
  block_sum2(before, total);
  const int64_t Ttot = (int64_t)A.Hkv * total;
  const int N = ctx_rows_of(A.ctx_start, A.ctx_len, bb, A.ctx_rows, A.max_prefix).len + A.S;
  const int64_t Ou = (int64_t)A.Hkv * before + (int64_t)g * N;
  const int wf = owner_of(Ou, Ttot, A.W), wl = owner_of(Ou + N - 1, Ttot, A.W);
  if (wf == wl) return;  // one workgroup held the whole unit and wrote the output itself
  const bool live = row < R;
  const int d = quad * VPT;
  float M = -INFINITY, L = 0.f;
  float acc[VPT];
#pragma unroll
  for (int e = 0; e < VPT; ++e) acc[e] = 0.f;
  for (int w0 = wf + sg; live && w0 <= wl; w0 += NSG * CB) {
    float2 ml[CB];
    u32x4 ov[CB];
#pragma unroll
    for (int k = 0; k < CB; ++k) {
      const int wk = w0 + NSG * k;
      const size_t slot = (size_t)wk + u;
      // a workgroup whose key range is empty (fewer keys than workgroups) wrote no partial
      if (wk <= wl && (int64_t)wk * Ttot / A.W < (int64_t)(wk + 1) * Ttot / A.W) {
        ml[k] = A.ws_ml[slot * R + row];
        ov[k] = *reinterpret_cast<const u32x4*>(
            A.ws_o + ((((slot * RW + row / 32) * (D / 8) + quad / 2) * 2 + quad % 2) * 32 + row % 32) * VPT);
      } else {
        ml[k] = make_float2(-INFINITY, 0.f);
        ov[k] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    float bm = M;
#pragma unroll
    for (int k = 0; k < CB; ++k) bm = fmaxf(bm, ml[k].x);
    const float rs = (M == -INFINITY) ? 0.f : tt_exp2(M - bm);
    L *= rs;
#pragma unroll
    for (int e = 0; e < VPT; ++e) acc[e] *= rs;
#pragma unroll
    for (int k = 0; k < CB; ++k) {
      const float wk = (ml[k].x == -INFINITY) ? 0.f : tt_exp2(ml[k].x - bm) * ml[k].y;
      L += wk;
      const PT* pv = reinterpret_cast<const PT*>(&ov[k]);
#pragma unroll
      for (int e = 0; e < VPT; ++e) acc[e] = fmaf((float)pv[e], wk, acc[e]);
    }
    M = bm;
  }
  if constexpr (NSG > 1) {
    __shared__ float gm[CB_RB][NSG][QB], gl[CB_RB][NSG][QB];
    __shared__ float ga[CB_RB][NSG][QB][VPT];
    gm[rr][sg][qq] = M;
    gl[rr][sg][qq] = L;
#pragma unroll
    for (int e = 0; e < VPT; ++e) ga[rr][sg][qq][e] = acc[e];
    __syncthreads();
    if (sg != 0) return;
    for (int q = 1; q < NSG; ++q) {
      const float m2 = gm[rr][q][qq];
      if (m2 == -INFINITY) continue;
      const float bm = fmaxf(M, m2);
      const float r1 = (M == -INFINITY) ? 0.f : tt_exp2(M - bm);
      const float r2 = tt_exp2(m2 - bm);
      L = L * r1 + gl[rr][q][qq] * r2;
#pragma unroll
      for (int e = 0; e < VPT; ++e) acc[e] = acc[e] * r1 + ga[rr][q][qq][e] * r2;
      M = bm;
    }
  }
  if (!live) return;
  const float inv = 1.f / L;
  const int s = row / G, hq = g * G + row % G;
  T* op = A.out + (((size_t)bb * A.S + s) * A.Hq + hq) * D + d;
  typedef T ovec __attribute__((ext_vector_type(VPT)));  // exactly this thread's VPT outputs
  ovec v;
#pragma unroll
  for (int e = 0; e < VPT; ++e) v[e] = (T)(acc[e] * inv);
  *reinterpret_cast<ovec*>(op) = v;
}

#ifndef TT_AT_MIN_KEYS
#define TT_AT_MIN_KEYS 128
#endif
constexpr int MIN_KEYS_PER_WG = TT_AT_MIN_KEYS;
constexpr int AT_TARGET_WG = 256;

template <typename T, int D, bool CAUSAL>
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
  // A multiple of the unit count: with equal sequence lengths every unit then starts at a
  // workgroup boundary, and no workgroup pays a second piece's loads and partial store (batch 1,
  // 2K prefix: 33 -> 32 workgroups, 15.8 -> 14.1 us). Ragged lengths keep the exact balance.
  if (W > U) W -= W % U;
  const size_t slots = (size_t)W + U;
  // partial rows are stored in whole 32-row tiles
  const size_t o_bytes = tt_align_up(slots * (size_t)((R + 31) / 32 * 32) * D * sizeof(PartT<T>), 256);
  const size_t need = o_bytes + tt_align_up(slots * R * sizeof(float2), 256);
  int st = tt_workspace_check(ws, ws_bytes, need);
  if (st != 0) return st < 0 ? st : TT_OK;
  if ((uintptr_t)ws % 256) return TT_ERR_ARG;
  Args<T, D> a;
  a.q = (const T*)q; a.kb = (const T*)kb; a.vb = (const T*)vb;
  a.kc = (const T*)kc; a.vc = (const T*)vc;
  a.ctx_start = cs; a.ctx_len = cl; a.out = (T*)out;
  a.ws_o = (PartT<T>*)ws;
  a.ws_ml = (float2*)((char*)ws + o_bytes);
  a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.ctx_rows = ctx_rows; a.max_prefix = max_prefix; a.W = W;
  a.c = scale * LOG2E;
  hipLaunchKernelGGL((attn_partial<T, D, CAUSAL>), dim3(W), dim3(AT_THREADS), 0, stream, a);
  if (tt_launch_status() != TT_OK) return TT_ERR_HIP;
  if (W > 1) {
    // slot groups per quad: enough to cover a unit's partials (about W / U + 1) in one batch
    constexpr int NQ = D / (16 / (int)sizeof(PartT<T>));
    constexpr int NSG_MAX = 4;
    const int rblocks = (R + CB_RB - 1) / CB_RB;
    if (W / U + 1 >= 16) {
      constexpr int QB = CB_THREADS / (CB_RB * NSG_MAX);
      hipLaunchKernelGGL((attn_combine<T, D, NSG_MAX>), dim3(U, rblocks, NQ / QB), dim3(CB_THREADS), 0,
                         stream, a);
    } else {
      constexpr int QB = CB_THREADS / CB_RB;
      hipLaunchKernelGGL((attn_combine<T, D, 1>), dim3(U, rblocks, NQ / QB), dim3(CB_THREADS), 0, stream,
                         a);
    }
    if (tt_launch_status() != TT_OK) return TT_ERR_HIP;
  }
  return TT_OK;
}


// Host checks shared by the two attention entry points; TT_OK to proceed.
int attn_check(const void* q, const void* k_blk, const void* v_blk, const void* k_ctx, const void* v_ctx,
               const int32_t* ctx_start, const int32_t* ctx_len, const void* out, int B, int S, int Hq,
               int Hkv, int D, int64_t ctx_rows, int max_prefix, float softmax_scale, int dtype,
               const size_t* workspace_bytes) {
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
  return TT_OK;
}

template <bool CAUSAL>
int attn_dispatch(const void* q, const void* k_blk, const void* v_blk, const void* k_ctx, const void* v_ctx,
                  const int32_t* ctx_start, const int32_t* ctx_len, void* out, int B, int S, int Hq, int Hkv,
                  int D, int64_t ctx_rows, int max_prefix, float softmax_scale, int dtype, void* workspace,
                  size_t* workspace_bytes, hipStream_t s) {
  if (dtype == TT_BF16) {
    if (D == 128) return launch<bf16, 128, CAUSAL>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, ctx_rows, max_prefix, softmax_scale, workspace, workspace_bytes, s);
    return launch<bf16, 64, CAUSAL>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, ctx_rows, max_prefix, softmax_scale, workspace, workspace_bytes, s);
  }
  if (D == 128) return launch<float, 128, CAUSAL>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, ctx_rows, max_prefix, softmax_scale, workspace, workspace_bytes, s);
  return launch<float, 64, CAUSAL>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, ctx_rows, max_prefix, softmax_scale, workspace, workspace_bytes, s);
}

// Appends the block's K/V rows to the cache and advances ctx_len: one workgroup per sequence b,
// 16-byte copies; every thread reads ctx_len[b] before the barrier, thread 0 updates it after. A
// sequence outside the caller's contract (negative start or length, length above max_prefix, or
// no room for S rows before ctx_rows) is left as it is: nothing written, ctx_len[b] unchanged.
constexpr int AP_THREADS = 256;
__global__ __launch_bounds__(AP_THREADS) void kv_append(const unsigned char* __restrict__ k_new,
                                                        const unsigned char* __restrict__ v_new,
                                                        unsigned char* __restrict__ k_ctx,
                                                        unsigned char* __restrict__ v_ctx,
                                                        const int32_t* __restrict__ ctx_start,
                                                        int32_t* __restrict__ ctx_len, int S, int Hkv,
                                                        int row_bytes, int64_t ctx_rows, int max_prefix) {
  const int b = blockIdx.x;
  const int32_t c0 = ctx_start[b], l0 = ctx_len[b];
  const int64_t r0 = (int64_t)c0 + l0;  // first new cache row of sequence b
  if (c0 < 0 || l0 < 0 || l0 > max_prefix || r0 + S > ctx_rows) return;  // the same for the workgroup
  const int gpr = row_bytes / 16;                          // 16-byte granules per row
  const int n = S * Hkv * gpr;
  for (int x = threadIdx.x; x < n; x += AP_THREADS) {
    const int gr = x % gpr, sg = x / gpr;
    const int g = sg % Hkv, s = sg / Hkv;
    const size_t src = (((size_t)b * S + s) * Hkv + g) * row_bytes + 16 * gr;
    const size_t dst = ((size_t)g * ctx_rows + r0 + s) * row_bytes + 16 * gr;
    *reinterpret_cast<u32x4*>(k_ctx + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
    *reinterpret_cast<u32x4*>(v_ctx + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
  }
  __syncthreads();
  if (threadIdx.x == 0) ctx_len[b] = l0 + S;
}

}  // namespace

extern "C" int tt_block_attn(const void* q, const void* k_blk, const void* v_blk, const void* k_ctx,
                             const void* v_ctx, const int32_t* ctx_start, const int32_t* ctx_len,
                             void* out, int B, int S, int Hq, int Hkv, int D, int64_t ctx_rows,
                             int max_prefix, float softmax_scale, int dtype, void* workspace,
                             size_t* workspace_bytes, void* stream) {
  const int st = attn_check(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, D, ctx_rows,
                            max_prefix, softmax_scale, dtype, workspace_bytes);
  if (st != TT_OK) return st;
  return attn_dispatch<false>(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, D, ctx_rows,
                              max_prefix, softmax_scale, dtype, workspace, workspace_bytes, (hipStream_t)stream);
}

extern "C" int tt_context_extend(const void* q, const void* k_new, const void* v_new, void* k_ctx, void* v_ctx,
                                 const int32_t* ctx_start, int32_t* ctx_len, void* out, int B, int S, int Hq,
                                 int Hkv, int D, int64_t ctx_rows, int max_prefix, float softmax_scale, int dtype,
                                 void* workspace, size_t* workspace_bytes, void* stream) {
  if (!k_ctx || !v_ctx) return TT_ERR_ARG;  // the new rows are appended to the cache
  int st = attn_check(q, k_new, v_new, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, D, ctx_rows,
                      max_prefix, softmax_scale, dtype, workspace_bytes);
  if (st != TT_OK) return st;
  if ((int64_t)max_prefix + S > ctx_rows) return TT_ERR_ARG;  // no room for any append
  hipStream_t s = (hipStream_t)stream;
  st = attn_dispatch<true>(q, k_new, v_new, k_ctx, v_ctx, ctx_start, ctx_len, out, B, S, Hq, Hkv, D, ctx_rows,
                           max_prefix, softmax_scale, dtype, workspace, workspace_bytes, s);
  if (st != TT_OK || workspace == nullptr) return st;  // an error, or a size query
  const int row_bytes = D * (dtype == TT_BF16 ? 2 : 4);
  hipLaunchKernelGGL(kv_append, dim3(B), dim3(AP_THREADS), 0, s, (const unsigned char*)k_new,
                     (const unsigned char*)v_new, (unsigned char*)k_ctx, (unsigned char*)v_ctx, ctx_start, ctx_len,
                     S, Hkv, row_bytes, ctx_rows, max_prefix);
  return tt_launch_status();
}
