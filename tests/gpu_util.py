"""Helpers of the GPU parity tests: uploads of synthetic inputs and the commit comparison.

Tolerances (the block step's stated bar):
  * attention output and logits: max |gpu - oracle| <= 1e-2 for bf16 inputs, 2e-5 for fp32;
  * predictions (argmax over identical fp32 logits) bit-exact;
  * commit decisions, tokens and mask words bit-exact, except positions whose oracle
    confidence lies within 1e-3 of gamma, and floor picks among confidences that tie to 1e-6
    (relative) at the k-th place; both sides round differently there (fp32 vs fp64 sums).
"""
import numpy as np
import torch

ATOL_BF16 = 1e-2
ATOL_F32 = 2e-5
GAMMA_BAND = 1e-3
TIE_REL = 1e-6


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


def check_commit_step(S, gamma, step, T, bits_before, tokens_before, gpu, ref):
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
            k = -(-len(masked) // (T - step))
            kth = confs[min(k, len(confs)) - 1]
            for i in diff:
                c = float(ref["conf"][b][i])
                near_gamma = abs(c - gamma) <= GAMMA_BAND
                near_tie = abs(c - kth) <= TIE_REL * max(abs(kth), 1e-30)
                assert near_gamma or near_tie, (b, i, c, gamma, cg, cr)
            exempt_blocks += 1
            continue
        assert int(gpu["mask_bits"][b]) == int(ref["mask_bits"][b])
        assert int(gpu["n_masked"][b]) == int(ref["n_masked"][b])
        assert list(gpu["tokens"][b]) == list(ref["tokens"][b]), b
    return exempt_blocks
