/*
 * tt.h — C ABI of the TwoTower denoiser block step on AMD CDNA4 (gfx950).
 *
 * One denoising step of a masked block ("Nemotron-Labs-TwoTower" wiki page, sections
 * "Architecture" and "Block-wise generation"): the block's queries attend, with grouped-query
 * heads, over [context-tower cache ; the block's own keys/values] with no mask (bidirectional
 * inside the block); an LM-head product turns the block's hidden states into vocabulary logits;
 * confidence unmasking commits every still-masked position whose top probability reaches gamma
 * and keeps the rest masked, with a floor that finishes the block within the step budget.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer to memory the caller owns, except
 *     `workspace_bytes`, which is a host pointer. The library keeps no pointer after it returns
 *     and has no mutable global state; calls on different streams do not interact, except that
 *     they must not share a workspace or an in/out buffer while both are in flight.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue work: TT_OK
 *     means "launched"; a device fault surfaces at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched. Any error return means
 *     nothing was launched and nothing was written.
 *   - `dtype` is TT_F32 (IEEE fp32 storage) or TT_BF16 (bfloat16 storage). Arithmetic is fp32
 *     (MFMA fp32 accumulation) in both cases; bf16 outputs are rounded to nearest-even.
 *   - Workspace protocol (calls that take one): with workspace == NULL the call stores the
 *     required byte count in *workspace_bytes, returns TT_OK and launches nothing. Otherwise
 *     *workspace_bytes must hold the size of `workspace` (>= the required size, else
 *     TT_ERR_WORKSPACE). The attention calls' workspace needs no initialisation and is scratch
 *     afterwards. The unmasking calls' workspace (tt_confidence_unmask, tt_unmask_sample,
 *     tt_lmhead_unmask) starts with arrival counters, 64 bytes apart, for the B blocks and the
 *     B*S rows: its first align256(64 * (B + B*S)) bytes must be zero at entry, every call leaves
 *     them zero, and the rest is scratch. So zero-fill such a workspace before its first use, and
 *     again before a call with a larger B * (S + 1) than the calls before it on that workspace
 *     (its counters then cover bytes that held records). It must be 256-byte aligned (else
 *     TT_ERR_ARG).
 */
#ifndef TT_H
#define TT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum tt_dtype { TT_F32 = 0, TT_BF16 = 1 };

/* Commit rules of an unmasking step (see tt_unmask_sample). */
enum tt_sampler_kind { TT_SAMPLER_CONFIDENCE = 0, TT_SAMPLER_PREDICT_NOISE = 1 };

typedef struct tt_sampler {
  int kind;            /* enum tt_sampler_kind */
  float gamma;         /* TT_SAMPLER_CONFIDENCE: commit threshold on the confidence */
  float temperature;   /* > 0: confidences are max softmax(logits / temperature); 1 = plain */
} tt_sampler;

enum tt_status {
  TT_OK = 0,
  TT_ERR_ARG = -1,          /* invalid argument (null pointer, bad size, NaN parameter, ...) */
  TT_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels implement (head_dim, S, dtype) */
  TT_ERR_WORKSPACE = -3,    /* workspace smaller than required */
  TT_ERR_HIP = -4           /* the HIP runtime reported an error at launch */
};

/*
 * tt_block_attn — denoiser block attention for one layer ("Nemotron-Labs-TwoTower" wiki page,
 * section "Architecture": the noisy block's queries attend over the context tower's layer-i
 * cache for the earlier blocks concatenated with the denoiser's own layer-i keys and values
 * for the current block; bidirectional inside the block, so no mask applies).
 *
 * For every sequence b, block position s and query head h (kv head g = h / (Hq/Hkv)):
 *   keys   = [ k_ctx[g][ctx_start[b] .. ctx_start[b]+ctx_len[b]) ; k_blk[b][0..S)[g] ]
 *   values = the same rows of v_ctx / v_blk
 *   out[b][s][h] = softmax(softmax_scale * keys . q[b][s][h]) . values
 *
 * Layouts (row-major, element = dtype):
 *   q, out       [B][S][Hq][D]
 *   k_blk, v_blk [B][S][Hkv][D]
 *   k_ctx, v_ctx [Hkv][ctx_rows][D]   (sequences packed along ctx_rows)
 *   ctx_start, ctx_len  int32 [B] on the device; ctx_len[b] may be 0.
 * Caller's contract: 0 <= ctx_start[b], 0 <= ctx_len[b] <= max_prefix and
 *   ctx_start[b] + ctx_len[b] <= ctx_rows. max_prefix sizes the launch. The kernels read both
 *   arrays through a clamp, in every build: start = ctx_start[b] within [0, ctx_rows], then
 *   len = ctx_len[b] within [0, min(max_prefix, ctx_rows - start)], and the output is the
 *   attention over those rows. Inside the contract this changes nothing; outside it no access
 *   leaves k_ctx / v_ctx.
 * Supported: D in {64, 128}; S*(Hq/Hkv) <= 256; dtype TT_F32 or TT_BF16.
 * Errors: TT_ERR_ARG for null pointers, B/S/Hq/Hkv <= 0, Hq % Hkv != 0, ctx_rows < 0,
 *   max_prefix < 0, max_prefix > 0 with null k_ctx/v_ctx, non-finite or non-positive scale;
 *   TT_ERR_UNSUPPORTED for D or S*G outside the supported set; TT_ERR_WORKSPACE; TT_ERR_HIP.
 * Workspace: split-K partial results (fp32), sized from B, Hkv, S*G, D and max_prefix.
 */
int tt_block_attn(const void* q, const void* k_blk, const void* v_blk,
                  const void* k_ctx, const void* v_ctx,
                  const int32_t* ctx_start, const int32_t* ctx_len,
                  void* out,
                  int B, int S, int Hq, int Hkv, int D, int64_t ctx_rows, int max_prefix,
                  float softmax_scale, int dtype,
                  void* workspace, size_t* workspace_bytes, void* stream);

/*
 * tt_context_extend — the context tower's attention step over a newly committed block, then the
 * append of its keys/values to the cache ("Nemotron-Labs-TwoTower" wiki page, section
 * "Block-wise generation": once a block is clean it is committed and the context tower processes
 * the committed tokens causally to update its caches; the context tower's attention is causal).
 *
 * For every sequence b, committed position s and query head h (kv head g = h / (Hq/Hkv)):
 *   keys   = [ k_ctx[g][ctx_start[b] .. ctx_start[b]+ctx_len[b]) ; k_new[b][0..s][g] ]
 *   values = the same rows of v_ctx / v_new
 *   out[b][s][h] = softmax(softmax_scale * keys . q[b][s][h]) . values
 * i.e. tt_block_attn with the block made causal (new row j visible to positions s >= j only).
 * Then, after the attention has read the cache: for j < S, cache row ctx_start[b]+ctx_len[b]+j
 * of kv head g receives k_new[b][j][g] (and v_new likewise), and ctx_len[b] += S.
 *
 * Layouts as tt_block_attn (k_new, v_new in the place of k_blk, v_blk); k_ctx, v_ctx and
 * ctx_len are updated in place. Caller's contract: that of tt_block_attn, and the S rows after
 * each sequence's cached rows are inside [0, ctx_rows) and belong to it (no other sequence's rows
 * there). The attention reads the lengths through the clamp of tt_block_attn. A sequence with
 * ctx_start[b] < 0, ctx_len[b] outside [0, max_prefix] or ctx_start[b] + ctx_len[b] + S > ctx_rows
 * gets no append: its cache rows and ctx_len[b] are left unchanged. Sizes, dtypes and limits as
 * tt_block_attn.
 * Errors: those of tt_block_attn; TT_ERR_ARG also for a null k_ctx / v_ctx, and when
 *   max_prefix + S > ctx_rows (no room to append).
 * Workspace: as tt_block_attn for the same arguments.
 */
int tt_context_extend(const void* q, const void* k_new, const void* v_new,
                      void* k_ctx, void* v_ctx,
                      const int32_t* ctx_start, int32_t* ctx_len,
                      void* out,
                      int B, int S, int Hq, int Hkv, int D, int64_t ctx_rows, int max_prefix,
                      float softmax_scale, int dtype,
                      void* workspace, size_t* workspace_bytes, void* stream);

/*
 * tt_lmhead_logits — vocabulary logits of every block position ("Nemotron-Labs-TwoTower" wiki
 * page, section "Block-wise generation": each step predicts all masked positions in parallel).
 *
 *   logits[m][v] = sum_k hidden[m][k] * w[v][k]        (no bias, no normalisation)
 *
 * Layouts: hidden [M][H] (dtype), w [V][H] (dtype), logits [M][V] fp32 (always fp32, so the
 * confidence test that follows sees full-precision logits).
 * Supported: H % 32 == 0; dtype TT_F32 or TT_BF16.
 * Errors: TT_ERR_ARG for null pointers or M, H, V <= 0; TT_ERR_UNSUPPORTED for H % 32 != 0 or
 *   an unknown dtype; TT_ERR_HIP.
 */
int tt_lmhead_logits(const void* hidden, const void* w, float* logits,
                     int M, int H, int V, int dtype, void* stream);

/*
 * tt_confidence_unmask — one confidence-unmasking step over B blocks ("Nemotron-Labs-TwoTower"
 * wiki page, section "Block-wise generation"; the operating point gamma = 0.8, S = 16, 16 steps
 * per block is given there; mask id 3 comes from the MLX port's configuration table).
 *
 * For each block b, with Mk = the positions whose bit is set in mask_bits[b] at entry:
 *   conf_i, pred_i = max and lowest argmax of softmax(logits row) with the mask id's logit
 *                    treated as -inf (so the mask token is never predicted), i in Mk;
 *   C = { i in Mk : conf_i >= gamma };   k = ceil(|Mk| / (num_steps - step));
 *   if |C| < k, C = the k most confident positions of Mk (ties: lower position first);
 *   tokens[b][i] = pred_i and bit i cleared for i in C; n_masked[b] = |Mk| - |C|.
 * Positions outside Mk are never read (their logits rows may hold anything) nor written.
 * Bits S..63 of a mask word name no position: they are ignored and stored back unchanged.
 * Layouts: logits fp32 [B*S][V] (row b*S+i is position i of block b); tokens int32 [B][S]
 *   (in/out); mask_bits uint64 [B] (in/out; bit i = position i still masked); n_masked int32 [B]
 *   (out). conf_out fp32 [B*S] and pred_out int32 [B*S] are optional (NULL = not written); when
 *   given they receive (conf_i, pred_i) for positions in Mk and (-1.0f, -1) for the others.
 * Supported: 1 <= S <= 64, V <= 2^31 - 4097.
 * Errors: TT_ERR_ARG for null required pointers, B <= 0, S <= 0, V < 2, mask_id outside
 *   [0, V), num_steps <= 0, step outside [0, num_steps), NaN gamma; TT_ERR_UNSUPPORTED for
 *   S > 64 or a larger V; TT_ERR_WORKSPACE; TT_ERR_HIP. Any finite or infinite gamma is legal (gamma > 1
 *   commits exactly the floor's k per step; gamma <= 0 commits every masked position).
 * Workspace: the arrival counters (zero at entry, zero again at exit; see the workspace
 *   protocol), then partial reductions of each row's vocabulary ranges and one per row, sized from
 *   B, S and V. The step is one kernel: the last workgroup of a row to finish merges the row, and
 *   the last row of a block to finish commits the block.
 */
int tt_confidence_unmask(const float* logits, int32_t* tokens, uint64_t* mask_bits,
                         int32_t* n_masked, float* conf_out, int32_t* pred_out,
                         int B, int S, int V, int step, int num_steps, float gamma, int mask_id,
                         void* workspace, size_t* workspace_bytes, void* stream);

/*
 * tt_confidence_unmask_noalloc — tt_confidence_unmask for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, results and errors as tt_confidence_unmask without the workspace: the call
 * keeps its arrival counters and partial reductions in a scratch array of 2 MiB that the library
 * holds on each device it runs on (until the process ends), and calls no allocator.
 * Limit: B + B * S <= 8192 (B * S <= 7696 at S = 16; the records then fit at any V); beyond it
 * the call returns TT_ERR_WORKSPACE and launches nothing. TT_ERR_HIP also when the scratch's
 * device address cannot be looked up. The counters have a fixed place in the scratch: they are
 * zero when the library is loaded and every call leaves them zero, whatever the sizes of the
 * calls before it.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's contents: calls
 * that overlap in time on one GPU (other streams, other host threads) race, and the caller must
 * serialise them.
 */
int tt_confidence_unmask_noalloc(const float* logits, int32_t* tokens, uint64_t* mask_bits,
                                 int32_t* n_masked, float* conf_out, int32_t* pred_out,
                                 int B, int S, int V, int step, int num_steps, float gamma,
                                 int mask_id, void* stream);

/*
 * tt_lmhead_unmask — tt_lmhead_logits followed by tt_confidence_unmask in one call, with the
 * vocabulary reduction done in the LM-head kernel's epilogue, so the [B*S][V] logits are never
 * stored ("Nemotron-Labs-TwoTower" wiki page, section "Block-wise generation": the step needs,
 * per masked position, only the top probability and its token).
 *
 * Computes what tt_unmask_sample (with the given host `sampler`) computes on the logits
 *   l[m][v] = sum_k hidden[m][k] * w[v][k]  (+ bias_val[m] when v == bias_tok[m])
 * for m = b*S + i. The optional bias adds one value to one vocabulary entry per row (a logit bias
 * such as a forced or banned token); bias_tok[m] outside [0, V) adds nothing. Both bias
 * pointers are NULL, or both are device arrays of B*S entries.
 * Layouts: hidden [B*S][H] bf16, w [V][H] bf16; tokens, mask_bits, n_masked, conf_out,
 *   pred_out as for tt_confidence_unmask (conf_out / pred_out optional).
 * Results: equal to the two-call path up to fp32 rounding order of the softmax sum (the logits
 *   themselves are the same fp32 accumulators); deterministic run to run.
 * Supported: dtype TT_BF16, H % 64 == 0, 1 <= S <= 64.
 * Errors: those of tt_unmask_sample; TT_ERR_ARG also for null hidden / w, H <= 0, exactly one
 *   bias pointer NULL, hidden or w not 16-byte aligned; TT_ERR_UNSUPPORTED for dtype TT_F32,
 *   H % 64 != 0 or S > 64.
 * Workspace: the arrival counters (as for tt_confidence_unmask), then one 16-byte record per
 *   (row, block of 16 to 128 vocabulary columns, by B*S and V) plus one per row, sized from B*S and V.
 */
int tt_lmhead_unmask(const void* hidden, const void* w, const int32_t* bias_tok,
                     const float* bias_val, int32_t* tokens, uint64_t* mask_bits,
                     int32_t* n_masked, float* conf_out, int32_t* pred_out,
                     int B, int S, int H, int V, int step, int num_steps,
                     const tt_sampler* sampler, int mask_id, int dtype, void* workspace,
                     size_t* workspace_bytes, void* stream);

/*
 * tt_unmask_sample — tt_confidence_unmask with a choice of sampler (the sampler variants of
 * "Nemotron-Labs-TwoTower" wiki page, section "Block-wise generation", and its model-card
 * example's temperature 0.1).
 *
 *   conf_i = max softmax(logits row / temperature) (mask id excluded), pred_i = its lowest
 *            argmax (temperature never changes pred_i);
 *   TT_SAMPLER_CONFIDENCE:    commit exactly as tt_confidence_unmask with this gamma (and
 *                             tt_confidence_unmask is this call with temperature 1);
 *   TT_SAMPLER_PREDICT_NOISE: the block-diffusion predict-and-noise sampler: with a linear noise
 *                             schedule, target = floor(S (num_steps - 1 - step) / num_steps)
 *                             positions stay masked after the step, so the
 *                             max(|Mk| - target, 0) most confident masked positions commit (ties:
 *                             lower position first); gamma is not used.
 * The schedule over S (not over the masked count) and its linearity are this library's reading:
 * the page names the sampler, not its schedule.
 * Arguments, layouts, workspace and errors as tt_confidence_unmask, plus: `sampler` is a HOST
 * pointer, read before the call returns; TT_ERR_ARG for a null sampler, a temperature that is
 * not finite and positive, or a NaN gamma; TT_ERR_UNSUPPORTED for an unknown kind.
 */
int tt_unmask_sample(const float* logits, int32_t* tokens, uint64_t* mask_bits,
                     int32_t* n_masked, float* conf_out, int32_t* pred_out,
                     int B, int S, int V, int step, int num_steps, const tt_sampler* sampler,
                     int mask_id, void* workspace, size_t* workspace_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* tt_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
int tt_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TT_H */
