"""End-to-end block runs on the GPU against the oracle's step composition, oracle.denoise_step.

A whole block is generated, T = 16 steps ("Nemotron-Labs-TwoTower" wiki page, section
"Block-wise generation": every step predicts all masked positions, commits the confident ones,
and the block finishes within the step budget). Each GPU step is
  tt_block_attn for every layer -> tt_lmhead_logits -> synthetic spikes -> tt_confidence_unmask
(the three-call step), and, beside it on its own block state, the fused step
  tt_block_attn for every layer -> tt_lmhead_unmask (spikes as its logit bias).

Every step of both paths is compared with denoise_step run from the state that path started the
step with (after an exempt divergence the oracle is re-seeded with the GPU's state):
  * attention outputs of every layer within 1e-2 of the oracle's at the first step, and bitwise
    the same at every later step (the inputs do not change within a block);
  * the three-call path stage-wise: its unmask equals the oracle's unmask of the GPU's own fp32
    logits bit for bit (up to the gamma band and floor ties);
  * both paths end to end against the oracle's fp64 logits, with the exemptions of
    gpu_util.check_fused_step;
  * both blocks finish: no mask bit left, no mask token emitted, n_masked strictly decreasing.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL_BF16, attn_dev, check_commit_step, check_fused_step, dev, host_bits

pytestmark = pytest.mark.gpu

bmd = pytest.importorskip("block_mask_diffusion_amd")


def _state(tok_d, bits_d, nm, conf, pred, B, S):
    return dict(tokens=tok_d.cpu().numpy(), mask_bits=host_bits(bits_d), n_masked=nm.cpu().numpy(),
                conf=conf.cpu().numpy().reshape(B, S), pred=pred.cpu().numpy().reshape(B, S))


def _run_block(wl):
    B, S, T = wl.B, wl.S, wl.T
    layers = [synth.attn_inputs(wl, l) for l in range(wl.layers)]
    layers_d = [attn_dev(x) for x in layers]
    lm = synth.lmhead_inputs(wl)
    sp = synth.spikes(wl)
    st = synth.initial_state(wl)
    hid_d, w_d = dev(lm["hidden"]), dev(lm["w"])
    spk_idx = torch.from_numpy(np.arange(wl.M, dtype=np.int64) * wl.V + sp["tok"]).cuda()
    spk_val = torch.from_numpy(sp["val"]).cuda()
    bt_d = torch.from_numpy(sp["tok"].astype(np.int32)).cuda()
    logits = torch.empty((wl.M, wl.V), dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(d["q"]) for d in layers_d]
    paths = {"three-call": dict(tok=dev(st["tokens"]), bits=dev(st["mask_bits"])),
             "fused": dict(tok=dev(st["tokens"]), bits=dev(st["mask_bits"]))}
    first_attn = None
    nm_hist = {k: [] for k in paths}
    oracle_cache = {}
    for step in range(T):
        for name, p in paths.items():
            tokens_h, bits_h = p["tok"].cpu().numpy(), host_bits(p["bits"])
            for d, o in zip(layers_d, outs):
                bmd.tt_block_attn(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["ctx_start"],
                                  d["ctx_len"], max_prefix=wl.max_prefix, softmax_scale=d["scale"], out=o)
            nm = torch.empty(B, dtype=torch.int32, device="cuda")
            conf = torch.empty(wl.M, dtype=torch.float32, device="cuda")
            pred = torch.empty(wl.M, dtype=torch.int32, device="cuda")
            if name == "three-call":
                bmd.tt_lmhead_logits(hid_d, w_d, logits)
                logits.view(-1).scatter_add_(0, spk_idx, spk_val)
                bmd.tt_confidence_unmask(logits, p["tok"], p["bits"], nm, step, T, wl.gamma, wl.mask_id, conf, pred)
            else:
                bmd.tt_lmhead_unmask(hid_d, w_d, p["tok"], p["bits"], nm, step, T, wl.gamma, wl.mask_id,
                                     bias_tok=bt_d, bias_val=spk_val, conf_out=conf, pred_out=pred)
            torch.cuda.synchronize()
            g = _state(p["tok"], p["bits"], nm, conf, pred, B, S)

            # the oracle's step from this path's starting state (shared when both paths agree)
            key = (tokens_h.tobytes(), bits_h.tobytes())
            if key not in oracle_cache:
                oracle_cache.clear()
                oracle_cache[key] = oracle.denoise_step(layers, lm["hidden"], lm["w"], wl.dtype, sp["tok"],
                                                        sp["val"], tokens_h, bits_h, S, step, T, wl.gamma,
                                                        wl.mask_id)
            ref = oracle_cache[key]

            got_attn = [o.float().cpu().numpy() for o in outs]
            if first_attn is None:
                for l, (ga, ra) in enumerate(zip(got_attn, ref["attn"])):
                    err = float(np.max(np.abs(ga.astype(np.float64) - ra)))
                    assert err <= ATOL_BF16, (l, err)
                first_attn = got_attn
            else:
                for ga, fa in zip(got_attn, first_attn):
                    assert np.array_equal(ga, fa)

            if name == "three-call":
                # stage-wise: the oracle's unmask of the GPU's own fp32 logits
                lg32 = logits.cpu().numpy()
                r32 = oracle.confidence_unmask(lg32, tokens_h, bits_h, S, step, T, wl.gamma, wl.mask_id)
                check_commit_step(S, wl.gamma, step, T, bits_h, tokens_h, g, r32)
            check_fused_step(S, wl.gamma, step, T, bits_h, g, ref, lambda m: ref["logits"][m], wl.mask_id, range(B))
            nm_hist[name].append(g["n_masked"].copy())
    for name, p in paths.items():
        bits = host_bits(p["bits"])
        tok = p["tok"].cpu().numpy()
        assert np.all(bits == 0), name
        assert np.all(tok != wl.mask_id), name
        hist = np.array(nm_hist[name])
        for b in range(B):
            live = hist[:, b][hist[:, b] > 0]
            assert np.all(np.diff(live) < 0), (name, b)
    return paths


def test_block_run_batch1_prefix2048():
    """The batch-1, 2048-token-prefix workload as specified: one attention layer, the full
    2688 x 131072 LM head, 16 steps."""
    _run_block(synth.workload(1))


def test_block_run_six_layers_reduced_prefix():
    """The six-layer, batch-4 workload with 4096-token prefixes in place of 131072 (so the oracle's
    six fp64 attention layers finish in seconds per step); full LM head."""
    wl = synth.workload(4, prefixes=[4096] * 4)
    wl.wid = 1400
    _run_block(wl)


def test_block_run_partly_committed_ragged():
    """Ragged prefixes with half the blocks partly committed at the start (the batch-8 workload's
    mask state on a smaller vocabulary and ragged lengths)."""
    wl = synth.workload(2, B=6, prefixes=[3000, 17, 900, 0, 2500, 64], V=8192, partial_init=True)
    wl.wid = 1401
    _run_block(wl)
