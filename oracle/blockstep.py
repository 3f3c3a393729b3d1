"""CPU oracle for the TwoTower denoiser block step (fp64 numpy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this module: only the test suite, the package smoke check and the benchmark's
CPU-baseline leg use it. It shares no code, header, table or helper with the HIP
path; the only thing both sides share is the seeded input module ``synth``.

What it computes, each function citing the passage it follows. Page names:
  [wiki]  "Nemotron-Labs-TwoTower" (aiwiki article summarising the paper and model card)
  [mlx]   "Nemotron TwoTower · MLX" (README of the Apple-Silicon port)
  [blog]  "Nemotron-TwoTower: Rethinking LLM Throughput via Decoupled Diffusion"

Every function is the plain definition (or, for the commit rule, the algorithm's
steps in the pages' order) in float64, with numpy's matmul/exp/max as the only
library steps. No blocking, splitting or reordering beyond the definitions.

Readings where the pages are silent (each also listed in the design notes):
  * softmax scale is an explicit argument (1/sqrt(D) in every workload);
  * grouped-query attention maps query head h to kv head floor(h / (Hq/Hkv));
  * Q and K arrive already position-encoded, so the step itself is position-agnostic;
  * confidence = the largest softmax probability at temperature 1, after the mask
    token's logit is set to -inf (so the mask token is never emitted);
  * the threshold test is ``conf >= gamma``;
  * the completion floor commits the k = ceil(n_masked / (T - step)) most confident
    masked positions when fewer than k clear gamma (ties: lower position first);
  * argmax ties go to the lowest vocabulary id;
  * the LM head is a bias-free product hidden . W^T with fp32 logits;
  * the context tower's step over a committed block: its new keys/values arrive as inputs
    (synthetic projections), attention is causal inside the block, and the new rows are
    appended right after each sequence's cached rows.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests
(brute force, closed forms, library special cases, invariants and a hand-worked
commit trace); see tests/test_oracle_*.py.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------- inputs

def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs: bf16 bit patterns (uint16) or float32."""
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- attention

def block_attention(inp: dict, dtype: str, rows: Optional[Iterable[Tuple[int, int, int]]] = None,
                    return_probs: bool = False):
    """Denoiser block attention ([wiki] "Architecture": the noisy block's queries attend over
    the concatenation of the context tower's layer-i cache for the earlier blocks and the
    denoiser's own layer-i keys/values for the current block; inside the block attention is
    bidirectional, so no mask applies anywhere).

    For sequence b, block position s, query head h, with kv head g = h // (Hq/Hkv):
        K = [K_ctx[g, start_b : start_b + len_b] ; K_blk[b, :, g]]   (V likewise)
        z = scale * K q_{b,s,h};  p = exp(z - max z) / sum exp(z - max z);  o = p^T V

    inp: dict from synth.attn_inputs (q [B][S][Hq][D], k_blk/v_blk [B][S][Hkv][D],
    k_ctx/v_ctx [Hkv][rows][D], ctx_start/ctx_len [B], scale).
    rows: optional iterable of (b, s, h); then returns {(b, s, h): o} (and probs).
    Otherwise returns o as float64 [B][S][Hq][D] (and probs per (b, g) if asked).
    """
    q = inp["q"]
    B, S, Hq, D = q.shape
    Hkv = inp["k_blk"].shape[2]
    G = Hq // Hkv
    scale = float(inp["scale"])
    starts = np.asarray(inp["ctx_start"], dtype=np.int64)
    lens = np.asarray(inp["ctx_len"], dtype=np.int64)

    def keys_values(b: int, g: int):
        a, n = int(starts[b]), int(lens[b])
        K = np.concatenate([decode(inp["k_ctx"][g, a:a + n], dtype), decode(inp["k_blk"][b, :, g], dtype)], axis=0)
        Vv = np.concatenate([decode(inp["v_ctx"][g, a:a + n], dtype), decode(inp["v_blk"][b, :, g], dtype)], axis=0)
        return K, Vv

    def attend(K, Vv, qvecs):
        z = scale * (qvecs @ K.T)                    # [rows][keys]
        z = z - z.max(axis=1, keepdims=True)
        e = np.exp(z)
        p = e / e.sum(axis=1, keepdims=True)
        return p @ Vv, p

    if rows is not None:
        want = {}
        for (b, s, h) in rows:
            want.setdefault((int(b), int(h) // G), []).append((int(b), int(s), int(h)))
        out, probs = {}, {}
        for (b, g), lst in want.items():
            K, Vv = keys_values(b, g)
            qv = np.stack([decode(q[bb, s, h], dtype) for (bb, s, h) in lst])
            o, p = attend(K, Vv, qv)
            for i, key in enumerate(lst):
                out[key] = o[i]
                probs[key] = p[i]
        return (out, probs) if return_probs else out

    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    probs = {}
    for b in range(B):
        for g in range(Hkv):
            K, Vv = keys_values(b, g)
            qg = decode(q[b, :, g * G:(g + 1) * G, :], dtype).reshape(S * G, D)
            o, p = attend(K, Vv, qg)
            out[b, :, g * G:(g + 1) * G, :] = o.reshape(S, G, D)
            probs[(b, g)] = p.reshape(S, G, -1)
    return (out, probs) if return_probs else out


def context_extend(inp: dict, dtype: str, rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """The context tower's step over a newly committed block ([wiki] "Block-wise generation": once
    a block is clean it is committed and the context tower processes the committed tokens
    causally to update its caches; [wiki] "Architecture" and [overview]: the context tower uses
    causal attention).

    inp: like block_attention's, with k_blk / v_blk holding the context tower's keys and values
    of the S committed tokens (k_new / v_new). For sequence b, position s, query head h, kv head
    g = h // (Hq/Hkv):
        K = [K_ctx[g, start_b : start_b + len_b] ; K_new[b, 0 .. s, g]]   (V likewise)
        o = softmax(scale * K q_{b,s,h}) V
    i.e. the prefix is visible to every new position and new row j only to positions s >= j.
    Then the new rows are appended: cache rows start_b + len_b + j (j < S) of kv head g get
    K_new[b, j, g] / V_new[b, j, g], and len_b grows by S.

    rows: optional iterable of (b, s, h): returns {(b, s, h): o} only (no cache update).
    Otherwise returns (o float64 [B][S][Hq][D], k_ctx', v_ctx' (copies, same dtype as given),
    ctx_len' int32 [B])."""
    q = inp["q"]
    B, S, Hq, D = q.shape
    Hkv = inp["k_blk"].shape[2]
    G = Hq // Hkv
    scale = float(inp["scale"])
    starts = np.asarray(inp["ctx_start"], dtype=np.int64)
    lens = np.asarray(inp["ctx_len"], dtype=np.int64)

    def attend(kpre: np.ndarray, vpre: np.ndarray, b: int, g: int, s: int, heads: Sequence[int]) -> np.ndarray:
        """Outputs of query heads `heads` (all in kv group g) at position s of sequence b, given
        that sequence's decoded prefix rows kpre / vpre of kv head g: each row is
        softmax(scale * K q) V over the prefix and new rows 0..s (the heads of one position see
        the same keys, so their score rows are one product)."""
        K = np.concatenate([kpre, decode(inp["k_blk"][b, :s + 1, g], dtype)], axis=0)
        Vv = np.concatenate([vpre, decode(inp["v_blk"][b, :s + 1, g], dtype)], axis=0)
        z = scale * (decode(q[b, s, heads], dtype) @ K.T)   # [heads][keys]
        e = np.exp(z - z.max(axis=1, keepdims=True))
        return (e / e.sum(axis=1, keepdims=True)) @ Vv

    want = {}
    if rows is not None:
        for (b, s, h) in rows:
            want.setdefault((int(b), int(h) // G), {}).setdefault(int(s), []).append(int(h))
    else:
        for b in range(B):
            for g in range(Hkv):
                want[(b, g)] = {s: list(range(g * G, (g + 1) * G)) for s in range(S)}
    got = {}
    for (b, g), by_s in want.items():
        a, n = int(starts[b]), int(lens[b])
        kpre = decode(inp["k_ctx"][g, a:a + n], dtype)
        vpre = decode(inp["v_ctx"][g, a:a + n], dtype)
        for s, heads in by_s.items():
            for h, o in zip(heads, attend(kpre, vpre, b, g, s, heads)):
                got[(b, s, h)] = o
    if rows is not None:
        return {(int(b), int(s), int(h)): got[(int(b), int(s), int(h))] for (b, s, h) in rows}
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    for (b, s, h), o in got.items():
        out[b, s, h] = o
    k_ctx = np.array(inp["k_ctx"], copy=True)
    v_ctx = np.array(inp["v_ctx"], copy=True)
    for b in range(B):
        r0 = int(starts[b] + lens[b])
        for j in range(S):
            k_ctx[:, r0 + j] = inp["k_blk"][b, j]
            v_ctx[:, r0 + j] = inp["v_blk"][b, j]
    return out, k_ctx, v_ctx, (lens + S).astype(np.int32)


# ----------------------------------------------------------------------------- LM head

def lmhead_logits(hidden: np.ndarray, w: np.ndarray, dtype: str) -> np.ndarray:
    """Vocabulary logits of every block position ([wiki] "Block-wise generation": each
    denoising step predicts all currently masked positions). logits = hidden . W^T, float64,
    with hidden [M][H] and W [V][H]; no bias, no norm (the pages name none)."""
    return decode(hidden, dtype) @ decode(w, dtype).T


def lmhead_entries(hidden: np.ndarray, w: np.ndarray, dtype: str,
                   pairs: Sequence[Tuple[int, int]]) -> np.ndarray:
    """Selected logits (m, v) of the same product, one dot product each."""
    return np.array([float(decode(hidden[m], dtype) @ decode(w[v], dtype)) for (m, v) in pairs])


# ----------------------------------------------------------------------------- confidence

def masked_softmax(row: np.ndarray, mask_id: int) -> np.ndarray:
    """Softmax of one logits row with the mask token excluded ([wiki] "Block-wise
    generation": predictions are constrained so the mask token itself is never emitted);
    the mask entry's logit becomes -inf, so its probability is 0."""
    l = np.array(row, dtype=np.float64)
    l[mask_id] = -np.inf
    m = l.max()
    e = np.exp(l - m)
    return e / e.sum()


def reduce_row(row: np.ndarray, mask_id: int, temperature: float = 1.0) -> Tuple[float, int]:
    """(confidence, prediction) of one position: the largest probability of the masked
    softmax and the lowest vocabulary id that attains it ([wiki] "Block-wise generation";
    [blog] "Adaptive Step-wise Generation"). With a temperature (the model card's diffusion
    example uses 0.1), the softmax is taken of logits / temperature; the prediction does not
    change."""
    l = np.array(row, dtype=np.float64)
    l[mask_id] = -np.inf
    m = l.max()
    a = int(np.flatnonzero(l == m)[0])
    s = float(np.exp((l - m) / float(temperature)).sum())
    return 1.0 / s, a


# ----------------------------------------------------------------------------- commit

def commit_block(conf: Sequence[float], pred: Sequence[int], tokens: np.ndarray, mask_bits: int,
                 S: int, step: int, T: int, gamma: float,
                 kind: str = "confidence") -> Tuple[np.ndarray, int, int, List[int]]:
    """One step of confidence unmasking for one block ([wiki] "Block-wise generation":
    every masked position is predicted in parallel; predictions whose confidence clears
    gamma are committed, the rest stay masked; a floor makes the block finish within T
    steps; decoded positions stay fixed).

    Steps, in order:
      masked set Mk = positions whose bit is set (empty: nothing changes, n_masked = 0)
      C = {i in Mk : conf_i >= gamma}
      k = ceil(|Mk| / (T - step))                      (the floor)
      if |C| < k: C = the k positions of Mk with the largest confidence (ties: lower i)
      for i in C: token_i = pred_i, clear bit i
      n_masked = |Mk| - |C|   (next step's timestep is n_masked / S)
    kind "predict_noise" is the block-diffusion sampler the wiki page mentions beside it (every
    masked position is predicted, then the lowest-confidence ones are re-masked as the noise
    schedule dictates): with a linear schedule, target = floor(S (T - 1 - step) / T) positions
    stay masked after the step, so C = the n_masked - target most confident masked positions
    (ties: lower i), none if n_masked <= target; gamma is not used.
    Returns (tokens, mask_bits, n_masked, committed positions)."""
    tokens = np.array(tokens, dtype=np.int32, copy=True)
    Mk = [i for i in range(S) if (mask_bits >> i) & 1]
    if not Mk:
        return tokens, mask_bits, 0, []
    if kind == "predict_noise":
        target = (S * (T - 1 - step)) // T
        k = max(len(Mk) - target, 0)
        C = sorted(Mk, key=lambda i: (-conf[i], i))[:k]
    elif kind == "confidence":
        C = [i for i in Mk if conf[i] >= gamma]
        k = -(-len(Mk) // (T - step))
        if len(C) < k:
            C = sorted(Mk, key=lambda i: (-conf[i], i))[:k]
    else:
        raise ValueError(kind)
    for i in sorted(C):
        tokens[i] = pred[i]
        mask_bits &= ~(1 << i)
    return tokens, mask_bits, len(Mk) - len(C), sorted(C)


def confidence_unmask(logits: np.ndarray, tokens: np.ndarray, mask_bits: np.ndarray, S: int,
                      step: int, T: int, gamma: float, mask_id: int, temperature: float = 1.0,
                      kind: str = "confidence"):
    """The whole unmask call over B blocks: logits [B*S][V] (any float dtype, read as float64),
    tokens int32 [B][S], mask_bits uint64 [B]. Rows of positions that are not masked at the
    start of the step are not read and keep their tokens.

    Returns dict(tokens, mask_bits, n_masked, conf, pred, committed) where conf/pred are
    (-1.0, -1) for positions not masked at step start."""
    B = tokens.shape[0]
    tok_out = np.array(tokens, dtype=np.int32, copy=True)
    bits_out = np.array(mask_bits, dtype=np.uint64, copy=True)
    n_masked = np.zeros(B, dtype=np.int32)
    conf = np.full((B, S), -1.0)
    pred = np.full((B, S), -1, dtype=np.int64)
    committed = []
    for b in range(B):
        bits = int(mask_bits[b])
        for i in range(S):
            if (bits >> i) & 1:
                c, a = reduce_row(logits[b * S + i], mask_id, temperature)
                conf[b, i], pred[b, i] = c, a
        t, nb, nm, C = commit_block(conf[b], pred[b], tokens[b], bits, S, step, T, gamma, kind)
        tok_out[b], bits_out[b], n_masked[b] = t, np.uint64(nb), nm
        committed.append(C)
    return dict(tokens=tok_out, mask_bits=bits_out, n_masked=n_masked, conf=conf, pred=pred,
                committed=committed)


# ----------------------------------------------------------------------------- one step

def denoise_step(attn_layers: Sequence[dict], hidden: np.ndarray, w: np.ndarray, dtype: str,
                 spike_tok: np.ndarray, spike_val: np.ndarray, tokens: np.ndarray,
                 mask_bits: np.ndarray, S: int, step: int, T: int, gamma: float, mask_id: int):
    """One denoiser block step as the benchmark runs it: block attention for every layer
    (outputs are returned; the synthetic workloads have no projections to chain them), the
    LM head, the synthetic logit spikes (an input-construction step, not part of the method),
    then confidence unmasking."""
    outs = [block_attention(inp, dtype) for inp in attn_layers]
    logits = lmhead_logits(hidden, w, dtype)
    logits[np.arange(logits.shape[0]), spike_tok] += spike_val.astype(np.float64)
    res = confidence_unmask(logits, tokens, mask_bits, S, step, T, gamma, mask_id)
    res["attn"] = outs
    res["logits"] = logits
    return res
