// LM-head product for more than 16 hidden rows, bf16 (on small vocabularies, up to 128 rows, the
// LDS-staged kernel of lmhead.hip runs instead) ("Nemotron-Labs-TwoTower" wiki page, section
// "Block-wise generation": every denoising step predicts all masked positions of every block in
// parallel). Up to a hundred-odd rows the W stream from HBM sets the pace; from a few hundred
// rows on, the matrix cores and the re-reads of the hidden rows from L2 do.
//
// Built with the iterative ILP machine scheduler (see build.py): with one wave per SIMD the
// kernel relies on the next k-step's LDS reads being in flight while the current MFMAs run,
// which the default occupancy-oriented schedule undoes by sinking each read next to its use.
#include "lmhead_int.h"
#include "reduce_int.h"

#include <type_traits>

namespace {

constexpr int LM_THREADS = 256;
constexpr int LM_WAVES = 4;
constexpr int NXCD = 8;
// v_mfma_f32_32x32x16_bf16 result layout (lane l, register j): column l % 32,
// row 8 (j / 4) + 4 (l / 32) + j % 4
__device__ __forceinline__ int mrow(int lane, int j) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

// Workgroup = 4 waves, one per SIMD, each owning a block of TM x TN MFMA 32x32x16 tiles (16 TM TN
// accumulators per lane, held in AGPRs). Both operands go HBM/L2 -> LDS by direct loads into a
// ring of GM_KB = 64-wide k stages, as deep as the LDS holds (up to 4): each row contributes one
// whole 128-byte line per stage, and the later stages' loads run while the current one is
// multiplied. LDS -> registers in MFMA operand layout: a lane reads 16 bytes = 8 consecutive h of
// one row; the 16-byte granules of row r are stored at slot g ^ ((r >> 1) & 7), so the 16 rows
// read by 16 consecutive lanes hit 16 distinct 16-byte bank groups. The next k-step's fragments
// are read while the current k-step's MFMAs run.
// Tiles (hidden rows x vocabulary rows): 64 x 256 (1 x 4 waves of 2 x 2 tiles) up to 64 rows,
// whose 40 KiB stages fit a 4-deep ring, so three stages of W stream ahead per CU (the product is
// HBM-bound there; measured at 64 rows: 119 against 129-134 us for the fused call with the
// 128 x 512 tile and its 2-deep ring); 128 x 512 (1 x 4 waves of 4 x 4) up to 128 rows; 256 x 256
// (2 x 2 waves of 4 x 4) beyond. With two hidden-row blocks the workgroups of one vocabulary tile
// have dispatch ids congruent modulo 8 (same XCD) and 8 apart, so W is fetched from HBM once
// (measured with FETCH_SIZE); the 64 x 256 tile over two blocks (65 to 128 rows) measured slower
// (175-193 against 129-142 us). A 512 x 128 tile (W read by one workgroup only) measured slower
// at 512 rows: it doubles the re-reads of the hidden rows from L2. Also measured and not faster
// at 512 rows: 32-wide stages in a 4- or 5-deep ring (TT_GEMM_KB=32 builds the variant), the LDS
// reads pinned between the MFMAs of the previous k-step, and a per-workgroup rotation of the
// k-stage order.
#ifndef TT_GM_NBUF
#define TT_GM_NBUF 4
#endif
constexpr int GM_KB = TT_GEMM_KB, GM_NBUF = TT_GM_NBUF;  // the deepest ring the LDS holds, up to this
constexpr int GM_ROWB = GM_KB * 2;                  // bytes per LDS row
constexpr int GM_KS = GM_KB / 16;                   // MFMA k-steps per stage
constexpr int GM_GPR = GM_KB / 8;                   // 16-byte granules per row
constexpr int GM_RPC = 1024 / GM_ROWB;              // rows per 1 KiB load chunk (64 lanes x 16 B)
static_assert(GM_KB == 32 || GM_KB == 64, "stage width");
static_assert(GM_KS % 2 == 0, "k-steps are pipelined in pairs");

// granule slot permutation of row r: the 16 rows read by 16 consecutive lanes (one 256-byte
// LDS bank sweep) land in 16 distinct 16-byte bank groups
__device__ __forceinline__ int gm_swz(int r) { return (r / (256 / GM_ROWB)) % GM_GPR; }

// WM waves along the hidden rows, 4 / WM along the vocabulary, each owning a block of TM x TN
// MFMA tiles (32 TM hidden rows x 32 TN vocabulary rows): tile BM = 32 TM WM hidden rows x
// BN = 32 TN (4 / WM) vocabulary rows.
// RED = false: store the fp32 logits. RED = true: reduce each row's logits over the wave's 128
// columns to one (max, lowest argmax, sum exp) record in red.parts[row][vtile * WN + wn]; the
// logits never reach memory.
template <int WM, int TM, int TN, bool RED>
__global__ __launch_bounds__(LM_THREADS, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void lmhead_gemm_kernel(
    const bf16* __restrict__ hidden, const bf16* __restrict__ w, float* __restrict__ logits, int M, int H,
    int V, int nvt, int nmb, TtRedArgs red) {
  constexpr int WN = LM_WAVES / WM;
  constexpr int GM_BM = 32 * TM * WM, GM_BN = 32 * TN * WN;
  constexpr int WROWS = 32 * TM, WCOLS = 32 * TN;  // one wave's block
  constexpr int ASTAGE = GM_BM * GM_ROWB, BSTAGE = GM_BN * GM_ROWB;  // bytes per stage
  constexpr int ACPW = ASTAGE / 1024 / LM_WAVES, BCPW = BSTAGE / 1024 / LM_WAVES;  // chunks per wave
  constexpr int PER_STAGE = ACPW + BCPW;  // load instructions per wave and stage
  // ring depth: as deep as the LDS of one workgroup holds, up to GM_NBUF
  constexpr int NBUF = GM_NBUF * (ASTAGE + BSTAGE) <= 160 * 1024 ? GM_NBUF : 160 * 1024 / (ASTAGE + BSTAGE);
  static_assert(NBUF >= 2 && (NBUF - 2) * PER_STAGE <= 63, "ring depth");
  typedef bf16x8 frag;
  __shared__ __attribute__((aligned(16))) unsigned char sa[NBUF][ASTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char sb[NBUF][BSTAGE];

  const int id = blockIdx.x;
  const int grp = id / (NXCD * nmb);
  const int rem = id - grp * NXCD * nmb;
  const int mblk = rem / NXCD;
  const int vtile = grp * NXCD + rem % NXCD;
  if (vtile >= nvt) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = mblk * GM_BM, v0 = vtile * GM_BN;

  // Fused mode with a mask, on the two-m-block tile: only the still-masked rows are multiplied.
  // Every workgroup compacts the masked rows (ascending) from the mask words itself, and its
  // m-block takes compacted rows [m0, m0 + BM); m-blocks past the last masked row exit. Tile row
  // r is hidden row rowmap[r]. (The 128-row tile has no LDS to spare and needs one m-block for
  // up to 128 rows anyway.)
  constexpr bool GATHER = RED && WM == 2;
  __shared__ int rowmap[GATHER ? GM_BM : 1];
  int nrows = M - m0;  // valid tile rows; rows past them re-read a valid row, results unused
  if constexpr (GATHER) {
    if (red.mask_bits) {
      __shared__ int scan[LM_THREADS];
      int base = 0;
      // only bits 0 .. S-1 name positions of a block; higher bits are ignored (a stray one would
      // name a row of the next block, or one past M)
      const uint64_t valid = red.S >= 64 ? ~0ull : ((1ull << red.S) - 1);
      for (int b0 = 0; b0 < red.B; b0 += LM_THREADS) {
        const int b = b0 + tid;
        uint64_t bits = b < red.B ? (red.mask_bits[b] & valid) : 0ull;
        const int c = __popcll(bits);
        scan[tid] = c;
        __syncthreads();
        for (int off = 1; off < LM_THREADS; off <<= 1) {  // inclusive scan of the counts
          const int x = tid >= off ? scan[tid - off] : 0;
          __syncthreads();
          scan[tid] += x;
          __syncthreads();
        }
        int k = base + scan[tid] - c;  // compacted index of block b's first masked row
        const int total = scan[LM_THREADS - 1];
        while (bits) {
          const int i = __builtin_ctzll(bits);
          bits &= bits - 1;
          if (k >= m0 && k < m0 + GM_BM) rowmap[k - m0] = b * red.S + i;
          ++k;
        }
        base += total;
        __syncthreads();  // scan[] is reused by the next chunk of blocks
      }
      nrows = base - m0;
    } else {
      for (int r = tid; r < GM_BM; r += LM_THREADS) rowmap[r] = min(m0 + r, M - 1);
    }
    __syncthreads();
    if (nrows <= 0) return;  // the same for every thread
  }
  auto hrow = [&](int r) { return GATHER ? rowmap[min(r, nrows - 1)] : min(m0 + r, M - 1); };

  // load sources: chunk c = wave * CPW + i covers tile rows [RPC c, RPC (c + 1)); lane -> row
  // RPC c + lane / GPR, LDS slot lane % GPR, which holds logical granule slot ^ swz(row). Rows
  // past M (or the masked rows) or V re-read a valid row (in bounds; results never stored).
  const bf16* asrc[ACPW];
  const bf16* bsrc[BCPW];
#pragma unroll
  for (int i = 0; i < ACPW; ++i) {
    const int r = (wave * ACPW + i) * GM_RPC + lane / GM_GPR;
    asrc[i] = hidden + (size_t)hrow(r) * H + 8 * ((lane % GM_GPR) ^ gm_swz(r));
  }
#pragma unroll
  for (int i = 0; i < BCPW; ++i) {
    const int r = (wave * BCPW + i) * GM_RPC + lane / GM_GPR;
    bsrc[i] = w + (size_t)min(v0 + r, V - 1) * H + 8 * ((lane % GM_GPR) ^ gm_swz(r));
  }
  // this wave's first LDS slot of stage buffer 0 in each ring; the rest are constant offsets
  const uint32_t a_lds = tt_lds_addr(&sa[0][wave * ACPW * 1024]);
  const uint32_t b_lds = tt_lds_addr(&sb[0][wave * BCPW * 1024]);
  const int nst = H / GM_KB;
  auto issue = [&](int st) {
    const int buf = st % NBUF, k0 = st * GM_KB;
    const uint32_t ab = a_lds + buf * ASTAGE, bb = b_lds + buf * BSTAGE;
    tt_static_for<ACPW>([&](auto i) { tt_dma16_at<i * 1024>(asrc[i] + k0, ab); });
    // W streams with the non-temporal policy (measured on MI355X: 155 -> 125 us at 128 rows,
    // 221 -> 202 us at 256; unchanged at 512, where the two m-blocks of a tile still share it)
    tt_static_for<BCPW>([&](auto i) { tt_dma16_at<i * 1024, true>(bsrc[i] + k0, bb); });
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int mt = 0; mt < TM; ++mt)
#pragma unroll
    for (int nt = 0; nt < TN; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.f;

  // fragments of k-step ks of the stage in buffer buf
  auto read_frags = [&](int buf, int ks, frag (&fa)[TM], frag (&fb)[TN]) {
    const unsigned char* a_s = sa[buf];
    const unsigned char* b_s = sb[buf];
    const int gsl = 2 * ks + hh;
#pragma unroll
    for (int t = 0; t < (TM > TN ? TM : TN); ++t) {
      if (t < TM) {
        const int ra = WROWS * wm + 32 * t + l32;
        fa[t] = *reinterpret_cast<const frag*>(a_s + ra * GM_ROWB + 16 * (gsl ^ gm_swz(ra)));
      }
      if (t < TN) {
        const int rb = WCOLS * wn + 32 * t + l32;
        fb[t] = *reinterpret_cast<const frag*>(b_s + rb * GM_ROWB + 16 * (gsl ^ gm_swz(rb)));
      }
    }
  };
  auto mma_step = [&](const frag (&fa)[TM], const frag (&fb)[TN]) {
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
#pragma unroll
      for (int nt = 0; nt < TN; ++nt)
        acc[mt][nt] = RED ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nt], fa[mt], acc[mt][nt], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt], fb[nt], acc[mt][nt], 0, 0, 0);
  };

  // Stage st: wait for this wave's loads of it (those of the NBUF - 2 later stages may still
  // be in flight), barrier (every wave's loads of stage st are in LDS and every wave has read
  // stage st - 1), refill stage st - 1's buffer with stage st + NBUF - 1, then GM_KS k-steps
  // with the fragments of step ks + 1 read during step ks.
#pragma unroll
  for (int e = 0; e < NBUF - 1; ++e)
    if (e < nst) issue(e);
  for (int st = 0; st < nst; ++st) {
    const int later = min(nst - 1 - st, NBUF - 2);  // stages issued after st, in flight
    tt_static_for<NBUF - 1>([&](auto n) {
      if (later == n) tt_wait_vmem<n * PER_STAGE>();
    });
    tt_lds_barrier();
    if (st + NBUF - 1 < nst) issue(st + NBUF - 1);
    const int buf = st % NBUF;
    frag fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    read_frags(buf, 0, fa0, fb0);
#pragma unroll
    for (int ks = 0; ks < GM_KS; ks += 2) {
      read_frags(buf, ks + 1, fa1, fb1);
      mma_step(fa0, fb0);
      if (ks + 2 < GM_KS) read_frags(buf, ks + 2, fa0, fb0);
      mma_step(fa1, fb1);
    }
  }

  if constexpr (RED) {
    // The fused path multiplies W by the hidden rows (operands swapped), so each accumulator
    // tile holds logits transposed: lane l, register j of tile (mt, nt) is hidden row
    // 32 mt + l % 32 and vocabulary id cb + 32 nt + 8 (j / 4) + 4 (l / 32) + j % 4. A lane thus
    // holds half of its row's WCOLS logits and lane l ^ 32 the other half: the row reduction runs
    // in registers, with one exchange between the two halves of the wave.
    constexpr int NVAL = 16 * TN, NG = NVAL / 8;  // logits per lane and row, in groups of 8
    const int cb = v0 + WCOLS * wn;  // first vocabulary id of the block
    if (cb >= V) return;
    const int part = vtile * WN + wn;
    // only blocks that hold the mask id, the vocabulary's end or some row's bias entry (a wave-
    // uniform test) pay for the per-entry checks
    const bool special = (red.mask_id >= cb && red.mask_id < cb + WCOLS) || (cb + WCOLS > V);
    int btok[TM];
    float bval[TM];
    bool hit = false;
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
      const int mc = hrow(WROWS * wm + 32 * mt + l32);
      btok[mt] = red.bias_tok ? red.bias_tok[mc] : -1;
      bval[mt] = red.bias_tok ? red.bias_val[mc] : 0.f;
      hit = hit || (btok[mt] >= cb && btok[mt] < cb + WCOLS);
    }
    // vocabulary id of v[k] below: increasing in k for a fixed lane
    auto vid = [&](int k) { return cb + 32 * (k >> 4) + 8 * ((k & 15) >> 2) + 4 * hh + (k & 3); };
    // three instances, so that the wave-uniform choice stays a branch: plain; one row's bias
    // entry may lie in the block (about one block in eight at 512 rows); mask id or vocabulary
    // end in the block (every check, rare)
    auto reduce_rows = [&](auto mode) {
      constexpr int MODE = decltype(mode)::value;
#pragma unroll
      for (int mt = 0; mt < TM; ++mt) {
        float v[NVAL];
#pragma unroll
        for (int nt = 0; nt < TN; ++nt)
#pragma unroll
          for (int j = 0; j < 16; ++j) v[16 * nt + j] = acc[mt][nt][j];
        if constexpr (MODE == 1) {
          // v[k] gets the bias where vid(k) == btok; compares kept in small groups (hoisted, their
          // masks overflow the scalar registers)
          const int rel = btok[mt] - vid(0);
#pragma unroll
          for (int k = 0; k < NVAL; ++k) {
            v[k] = (rel == vid(k) - vid(0)) ? v[k] + bval[mt] : v[k];
            if ((k & 7) == 7) __builtin_amdgcn_sched_barrier(0);
          }
        } else if constexpr (MODE == 2) {
          // as above, then the mask id and ids past the vocabulary's end become -inf
          const int rel = btok[mt] - vid(0), relm = red.mask_id - vid(0), relv = V - vid(0);
#pragma unroll
          for (int k = 0; k < NVAL; ++k) {
            const int d = vid(k) - vid(0);
            const float x = (rel == d) ? v[k] + bval[mt] : v[k];
            v[k] = (relm == d || d >= relv) ? -INFINITY : x;
            if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);
          }
        }
        float mx[NG];
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          mx[q] = v[8 * q];
#pragma unroll
          for (int e = 1; e < 8; ++e) mx[q] = fmaxf(mx[q], v[8 * q + e]);
        }
#pragma unroll
        for (int w2 = NG / 2; w2 >= 1; w2 >>= 1)
#pragma unroll
          for (int q = 0; q < w2; ++q) mx[q] = fmaxf(mx[q], mx[q + w2]);
        const float rm = fmaxf(mx[0], tt_swap_halves(mx[0]));
        const bool empty = (rm == -INFINITY);
        const float mb = empty ? 0.f : rm * red.c;
        int kf = NVAL;  // first k (lowest id) of this lane holding the maximum; NVAL = none
#pragma unroll
        for (int k = NVAL - 1; k >= 0; --k) {
          kf = (v[k] == rm) ? k : kf;
          // keeps the compares next to their selects: hoisted, their masks overflow the SGPRs
          if ((k & 7) == 0) __builtin_amdgcn_sched_barrier(0);
        }
        int key = (kf < NVAL) ? vid(kf) : INT32_MAX;
        float sm[NG];
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          sm[q] = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sm[q] += tt_exp2(fmaf(v[8 * q + e], red.c, -mb));
        }
#pragma unroll
        for (int w2 = NG / 2; w2 >= 1; w2 >>= 1)
#pragma unroll
          for (int q = 0; q < w2; ++q) sm[q] += sm[q + w2];
        const float rs = sm[0] + tt_swap_halves(sm[0]);  // same sum on both halves (commutative)
        key = min(key, tt_swap_halves_i(key));
        const int rr = WROWS * wm + 32 * mt + l32;
        if (hh == 0 && rr < nrows) {
          const int m = GATHER ? rowmap[rr] : m0 + rr;
          TtPartial p;
          p.m = rm;
          p.s = rs;
          p.a = empty ? INT32_MAX : key;
          p.pad = 0;
          red.parts[(size_t)m * red.nparts + part] = p;
        }
      }
    };
    if (special) reduce_rows(std::integral_constant<int, 2>{});
    else if (__any(hit)) reduce_rows(std::integral_constant<int, 1>{});
    else reduce_rows(std::integral_constant<int, 0>{});
  } else {
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
#pragma unroll
      for (int nt = 0; nt < TN; ++nt) {
        const int v = v0 + WCOLS * wn + 32 * nt + l32;
        if (v >= V) continue;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = m0 + WROWS * wm + 32 * mt + mrow(lane, j);
          if (m < M) logits[(size_t)m * V + v] = acc[mt][nt][j];
        }
      }
  }
}


template <int WM, int TM, int TN, bool RED>
int gemm_launch(const void* hidden, const void* w, float* logits, int M, int H, int V, TtRedArgs red,
                hipStream_t s) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * (LM_WAVES / WM);
  const int nvt = (V + BN - 1) / BN;
  const int nmb = (M + BM - 1) / BM;
  const unsigned grid = (unsigned)(((nvt + NXCD - 1) / NXCD) * NXCD * nmb);
  hipLaunchKernelGGL((lmhead_gemm_kernel<WM, TM, TN, RED>), dim3(grid), dim3(LM_THREADS), 0, s, (const bf16*)hidden,
                     (const bf16*)w, logits, M, H, V, nvt, nmb, red);
  return tt_launch_status();
}

}  // namespace

// Tile by M (measured at H = 2688, V = 131072): up to 64 hidden rows, 64 x 256 tiles, whose
// 40 KiB stages leave room for a 4-deep ring (three stages of W in flight per CU); up to 128 rows,
// 128 x 512 tiles (W read once, few re-reads of the hidden rows); beyond, 256 x 256 (two
// hidden-row blocks share W in L2). On a vocabulary of 32768 or less the 128 x 512 tiles give 64
// workgroups or fewer, and the 256 x 256 tile, with twice as many, is faster at any M (128 rows,
// V = 32768: 78.6 against 94.7 us). Each output is the same chain of MFMAs in any tile.
enum GemmCfg { GM_256x256, GM_128x512, GM_64x256 };
GemmCfg gemm_cfg(int M, int V) {
  if ((V + 511) / 512 <= 64 || M > 128) return GM_256x256;
  return M <= 64 ? GM_64x256 : GM_128x512;
}

int tt_lm_gemm_cols(int M, int V) { return gemm_cfg(M, V) == GM_64x256 ? 64 : 128; }

int tt_lm_gemm_launch(const void* hidden, const void* w, float* logits, int M, int H, int V, hipStream_t s) {
  const TtRedArgs none{nullptr, nullptr, -1, nullptr, 0};
  switch (gemm_cfg(M, V)) {
    case GM_64x256: return gemm_launch<1, 2, 2, false>(hidden, w, logits, M, H, V, none, s);
    case GM_128x512: return gemm_launch<1, 4, 4, false>(hidden, w, logits, M, H, V, none, s);
    default: return gemm_launch<2, 4, 4, false>(hidden, w, logits, M, H, V, none, s);
  }
}

// Fused variant: per-(row, column block of one wave) reduction records instead of logits;
// red.nparts must be ceil(V / tt_lm_gemm_cols(M, V)).
int tt_lm_gemm_reduce_launch(const void* hidden, const void* w, int M, int H, int V, TtRedArgs red,
                             hipStream_t s) {
  switch (gemm_cfg(M, V)) {
    case GM_64x256: return gemm_launch<1, 2, 2, true>(hidden, w, nullptr, M, H, V, red, s);
    case GM_128x512: return gemm_launch<1, 4, 4, true>(hidden, w, nullptr, M, H, V, red, s);
    default: return gemm_launch<2, 4, 4, true>(hidden, w, nullptr, M, H, V, red, s);
  }
}
