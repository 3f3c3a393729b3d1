"""Helpers of the GPU parity tests: uploads of synthetic inputs and the commit comparison.

Tolerances (the block step's stated bar):
  * attention output and logits: max |gpu - oracle| <= 1e-2 for bf16 inputs, 2e-5 for fp32;
  * predictions (argmax over identical fp32 logits) bit-exact;
  * commit decisions, tokens and mask words bit-exact, except positions whose oracle
    confidence lies within 1e-3 of gamma, and floor picks among confidences that tie to 1e-6
    (relative) at the k-th place; both sides round differently there (fp32 vs fp64 sums).

The fused LM head + unmask call is compared with the oracle's fp64 logits (no logits are
stored to compare stage-wise), so its argmax is decided on fp32 accumulations on one side and
fp64 products on the other:
  * predictions bit-exact, except where the oracle's logit at the GPU's pick is within 1e-4
    of the row maximum (fp32 accumulation of H = 2688 products errs by about 1e-6 here): both
    are then argmaxes within the precision, and the pick is checked to be such a near-maximum;
  * confidences within 1e-2 absolute (the stated bar for floating point) and within
    CONF_REL_FUSED / temperature relative. conf = 1 / sum_v exp((l_v - l_max) / temperature), so
    a logit error of at most e moves log conf by at most 2 e / temperature; fp32 accumulation of
    2688 bf16 products (each exact in fp32) of a logit near N(0, 1) errs by a few 1e-6, so 1e-4
    leaves a margin of more than 3 over the worst case of that estimate;
  * commits as above, the floor's tie band being that same relative band (a floor pick is
    exempt only when its oracle confidence and the k-th largest one agree to within it).
"""
import numpy as np
import torch

ATOL_BF16 = 1e-2
ATOL_F32 = 2e-5
GAMMA_BAND = 1e-3
TIE_REL = 1e-6
PRED_TIE = 1e-4
CONF_REL_FUSED = 1e-4


def dev(x: np.ndarray, dtype: str = None) -> torch.Tensor:
    """Upload a synth array: uint16 bf16 bits -> torch.bfloat16, others as they are."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    if x.dtype == np.uint64:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int64)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def attn_dev(inp: dict) -> dict:
    return {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}


def committed(before: int, after: int, S: int):
    return [i for i in range(S) if (before >> i) & 1 and not (after >> i) & 1]


def floor_k(kind, n, S, step, T):
    """Number of positions the step must commit at least: the completion floor (confidence
    sampler) or the noise schedule's count (predict-and-noise)."""
    if kind == "predict_noise":
        return max(n - (S * (T - 1 - step)) // T, 0)
    return -(-n // (T - step))


def check_commit_step(S, gamma, step, T, bits_before, tokens_before, gpu, ref, kind="confidence"):
    """Compare one unmask step. gpu/ref: dicts with tokens [B][S], mask_bits [B] (uint64),
    n_masked [B], conf [B][S], pred [B][S]. Returns the number of blocks with an exempt
    divergence (0 when bit-exact). Raises AssertionError on a non-exempt difference."""
    B = tokens_before.shape[0]
    exempt_blocks = 0
    for b in range(B):
        before = int(bits_before[b])
        for i in range(S):
            if (before >> i) & 1:
                assert int(gpu["pred"][b][i]) == int(ref["pred"][b][i]), (b, i)
                rc, gc = float(ref["conf"][b][i]), float(gpu["conf"][b][i])
                assert abs(gc - rc) <= 1e-5 * rc + 1e-9, (b, i, gc, rc)
            else:
                assert int(gpu["conf"][b][i]) == -1 and int(gpu["pred"][b][i]) == -1
        cg = committed(before, int(gpu["mask_bits"][b]), S)
        cr = committed(before, int(ref["mask_bits"][b]), S)
        if cg != cr:
            diff = set(cg) ^ set(cr)
            masked = [i for i in range(S) if (before >> i) & 1]
            confs = sorted((float(ref["conf"][b][i]) for i in masked), reverse=True)
            k = floor_k(kind, len(masked), S, step, T)
            kth = confs[min(max(k, 1), len(confs)) - 1]
            for i in diff:
                c = float(ref["conf"][b][i])
                near_gamma = kind == "confidence" and abs(c - gamma) <= GAMMA_BAND
                near_tie = abs(c - kth) <= TIE_REL * max(abs(kth), 1e-30)
                assert near_gamma or near_tie, (b, i, c, gamma, cg, cr)
            exempt_blocks += 1
            continue
        assert int(gpu["mask_bits"][b]) == int(ref["mask_bits"][b])
        assert int(gpu["n_masked"][b]) == int(ref["n_masked"][b])
        assert list(gpu["tokens"][b]) == list(ref["tokens"][b]), b
    return exempt_blocks


def check_fused_step(S, gamma, step, T, bits_before, gpu, ref, logits_of, mask_id, blocks, kind="confidence",
                     temperature=1.0):
    """Compare one fused LM-head + unmask step on the given blocks. logits_of(row) returns the
    oracle's fp64 logits row (bias included). Returns (number of blocks with an exempt commit
    divergence, relative confidence errors of all masked positions checked)."""
    band = CONF_REL_FUSED / temperature
    exempt_blocks = 0
    rel = []
    for b in blocks:
        before = int(bits_before[b])
        alt = set()
        for i in range(S):
            if (before >> i) & 1:
                gp, rp = int(gpu["pred"][b][i]), int(ref["pred"][b][i])
                if gp != rp:
                    row = logits_of(b * S + i)
                    assert 0 <= gp < row.shape[0] and gp != mask_id, (b, i, gp)
                    assert row[rp] - row[gp] <= PRED_TIE, (b, i, gp, rp, row[rp] - row[gp])
                    alt.add(i)
                rc, gc = float(ref["conf"][b][i]), float(gpu["conf"][b][i])
                assert abs(gc - rc) <= ATOL_BF16, (b, i, gc, rc)
                assert abs(gc - rc) <= band * rc, (b, i, gc, rc, abs(gc - rc) / rc)
                rel.append(abs(gc - rc) / rc)
            else:
                assert int(gpu["conf"][b][i]) == -1 and int(gpu["pred"][b][i]) == -1
        cg = committed(before, int(gpu["mask_bits"][b]), S)
        cr = committed(before, int(ref["mask_bits"][b]), S)
        if cg != cr:
            masked = [i for i in range(S) if (before >> i) & 1]
            confs = sorted((float(ref["conf"][b][i]) for i in masked), reverse=True)
            k = floor_k(kind, len(masked), S, step, T)
            kth = confs[min(max(k, 1), len(confs)) - 1]
            for i in set(cg) ^ set(cr):
                c = float(ref["conf"][b][i])
                near_gamma = kind == "confidence" and abs(c - gamma) <= GAMMA_BAND
                assert near_gamma or abs(c - kth) <= band * kth, (b, i, c, gamma, cg, cr)
            exempt_blocks += 1
            continue
        assert int(gpu["mask_bits"][b]) == int(ref["mask_bits"][b])
        assert int(gpu["n_masked"][b]) == int(ref["n_masked"][b])
        for i in range(S):
            if i in alt:
                assert int(gpu["tokens"][b][i]) == int(gpu["pred"][b][i] if i in cg else ref["tokens"][b][i])
            else:
                assert int(gpu["tokens"][b][i]) == int(ref["tokens"][b][i]), (b, i)
    return exempt_blocks, rel
