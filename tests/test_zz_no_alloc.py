"""tt_confidence_unmask_noalloc (the unmasking step on the library's per-device scratch, for
callers that cannot allocate) against tt_confidence_unmask on the same inputs: two calls in a row,
the second smaller than the first, both bit for bit equal to the workspace call."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev, host_bits

pytestmark = pytest.mark.gpu

bmd = pytest.importorskip("block_mask_diffusion_amd")


def _both(wl, logits_np, step):
    st = synth.initial_state(wl)
    lg = dev(logits_np)
    out = []
    for fn in (bmd.tt_confidence_unmask, bmd.tt_confidence_unmask_noalloc):
        tok, bits = dev(st["tokens"]), dev(st["mask_bits"])
        nm = torch.full((wl.B,), -7, dtype=torch.int32, device="cuda")
        conf = torch.empty(wl.M, dtype=torch.float32, device="cuda")
        pred = torch.empty(wl.M, dtype=torch.int32, device="cuda")
        fn(lg, tok, bits, nm, step, wl.T, wl.gamma, wl.mask_id, conf, pred)
        torch.cuda.synchronize()
        out.append(dict(tok=tok.cpu().numpy(), bits=host_bits(bits), nm=nm.cpu().numpy(),
                        conf=conf.cpu().numpy().view(np.uint32), pred=pred.cpu().numpy()))
    return out


def test_noalloc_equals_the_workspace_call_twice_in_a_row():
    # first call: 48 blocks of 16 over the full vocabulary (1536 rows, 1.5 MiB of records);
    # second: 3 blocks of 16, partly committed, over a ragged vocabulary
    big = synth.workload(2, B=48, partial_init=True)
    big.wid = 1500
    small = synth.workload(2, B=3, V=5000, partial_init=True)
    small.wid = 1501
    for wl, step in ((big, 0), (small, 5)):
        ref, got = _both(wl, synth.direct_logits(wl), step)
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (wl.B, k)


def test_noalloc_rejects_sizes_past_its_scratch():
    wl = synth.workload(1, B=482, V=4096)   # 482 + 482 * 16 = 8194 counters > 8192
    st = synth.initial_state(wl)
    lg = torch.zeros((wl.M, wl.V), dtype=torch.float32, device="cuda")
    nm = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    with pytest.raises(bmd.TTError) as e:
        bmd.tt_confidence_unmask_noalloc(lg, dev(st["tokens"]), dev(st["mask_bits"]), nm, 0, 16, 0.8, 3)
    assert e.value.status == -3


def test_noalloc_at_its_largest_size_then_small_again():
    # 481 blocks of 16 (481 + 7696 = 8177 counters, the most that fit), then 2 blocks of 16 whose
    # rows are split into 32 ranges: the counters of the second call lie where the first call's did
    for wl in (synth.workload(2, B=481, V=4096), synth.workload(2, B=2, partial_init=True)):
        wl.wid = 1600 + wl.B
        ref, got = _both(wl, synth.direct_logits(wl), 0)
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (wl.B, k)
