"""CPU oracle (fp64 numpy) for the TwoTower denoiser block step.

Test infrastructure: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it. The product path never does."""
from .blockstep import (decode, block_attention, context_extend, lmhead_logits, lmhead_entries,
                        masked_softmax, reduce_row, commit_block, confidence_unmask, denoise_step)

__all__ = ["decode", "block_attention", "context_extend", "lmhead_logits", "lmhead_entries",
           "masked_softmax", "reduce_row", "commit_block", "confidence_unmask", "denoise_step"]
