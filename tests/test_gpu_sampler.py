"""GPU parity of the sampler variants against the oracle: tt_unmask_sample (temperature-scaled
confidence, predict-and-noise; block sizes 8 / 32 / 64) stage-wise on synth logits, and the fused
tt_lmhead_unmask with the same samplers against the oracle's fp64 LM head."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_commit_step, check_fused_step, dev, host_bits

pytestmark = pytest.mark.gpu

bmd = pytest.importorskip("block_mask_diffusion_amd")


def _gpu_step(logits_d, tokens_d, bits_d, S, step, T, mask_id, kind, gamma, tau):
    B = tokens_d.shape[0]
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    conf = torch.empty(B * S, dtype=torch.float32, device="cuda")
    pred = torch.empty(B * S, dtype=torch.int32, device="cuda")
    bmd.tt_unmask_sample(logits_d, tokens_d, bits_d, nm, step, T, mask_id, sampler=kind, gamma=gamma,
                         temperature=tau, conf_out=conf, pred_out=pred)
    torch.cuda.synchronize()
    return dict(tokens=tokens_d.cpu().numpy(), mask_bits=host_bits(bits_d), n_masked=nm.cpu().numpy(),
                conf=conf.cpu().numpy().reshape(B, S), pred=pred.cpu().numpy().reshape(B, S))


def _run(wl, logits, steps, kind, tau, gamma=None):
    gamma = wl.gamma if gamma is None else gamma
    st = synth.initial_state(wl)
    tokens_h, bits_h = st["tokens"].copy(), st["mask_bits"].copy()
    logits_d, tokens_d, bits_d = dev(logits), dev(tokens_h), dev(bits_h)
    exempt = 0
    for step in range(steps):
        ref = oracle.confidence_unmask(logits, tokens_h, bits_h, wl.S, step, wl.T, gamma, wl.mask_id, tau, kind)
        g = _gpu_step(logits_d, tokens_d, bits_d, wl.S, step, wl.T, wl.mask_id, kind, gamma, tau)
        exempt += check_commit_step(wl.S, gamma, step, wl.T, bits_h, tokens_h, g, ref, kind)
        tokens_h, bits_h = ref["tokens"], ref["mask_bits"]
        tokens_d.copy_(dev(tokens_h))
        bits_d.copy_(dev(bits_h))
    return exempt, tokens_h, bits_h


@pytest.mark.parametrize("tau", [0.1, 0.5, 2.0])
def test_temperature_confidence_full_vocab(tau):
    wl = synth.workload(1, B=2)
    wl.wid = 1100 + int(10 * tau)
    logits = synth.direct_logits(wl)
    _run(wl, logits, 3, "confidence", tau)


@pytest.mark.parametrize("tau", [1.0, 0.1])
def test_predict_noise_full_block(tau):
    wl = synth.workload(0, B=3)
    wl.wid = 1110 + int(10 * tau)
    logits = synth.direct_logits(wl)
    _, tokens, bits = _run(wl, logits, wl.T, "predict_noise", tau)
    assert np.all(bits == 0) and np.all(tokens != wl.mask_id)


def test_predict_noise_partial_blocks_and_short_schedule():
    wl = synth.workload(2, B=4, V=4096)
    wl.wid = 1120
    wl.T = 4
    logits = synth.direct_logits(wl)
    _, tokens, bits = _run(wl, logits, wl.T, "predict_noise", 1.0)
    assert np.all(bits == 0)


@pytest.mark.parametrize("S", [8, 32, 64])
@pytest.mark.parametrize("kind", ["confidence", "predict_noise"])
def test_block_sizes(S, kind):
    wl = synth.workload(0, S=S, B=2, V=2048)
    wl.wid = 1130 + S
    logits = synth.direct_logits(wl)
    _, tokens, bits = _run(wl, logits, wl.T, kind, 0.1)
    assert np.all(bits == 0) and np.all(tokens != wl.mask_id)


def test_temperature_one_equals_confidence_unmask_bitwise():
    wl = synth.workload(1, B=4)
    wl.wid = 1140
    logits = dev(synth.direct_logits(wl))
    st = synth.initial_state(wl)
    outs = []
    for f in ("sample", "plain"):
        tok, bits = dev(st["tokens"]), dev(st["mask_bits"])
        nm = torch.empty(wl.B, dtype=torch.int32, device="cuda")
        conf = torch.empty(wl.M, device="cuda")
        pred = torch.empty(wl.M, dtype=torch.int32, device="cuda")
        if f == "sample":
            bmd.tt_unmask_sample(logits, tok, bits, nm, 0, wl.T, wl.mask_id, gamma=wl.gamma, conf_out=conf,
                                 pred_out=pred)
        else:
            bmd.tt_confidence_unmask(logits, tok, bits, nm, 0, wl.T, wl.gamma, wl.mask_id, conf, pred)
        torch.cuda.synchronize()
        outs.append((tok.cpu().numpy(), bits.cpu().numpy(), conf.cpu().numpy().view(np.uint32), pred.cpu().numpy()))
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("B,kind,tau", [(1, "confidence", 0.1), (4, "predict_noise", 1.0), (12, "confidence", 0.1),
                                        (12, "predict_noise", 0.1)])
def test_fused_with_sampler(B, kind, tau):
    """The fused LM head + unmask call with the sampler variants (every hidden-row bucket)."""
    wl = synth.workload(1, B=B, H=128, V=3000)
    wl.wid = 1150 + B
    inp = synth.lmhead_inputs(wl)
    sp = synth.spikes(wl)
    bt, bv = sp["tok"].astype(np.int32), sp["val"]
    lg = oracle.lmhead_logits(inp["hidden"], inp["w"], "bf16")
    lg[np.arange(wl.M), bt] += bv.astype(np.float64)
    st = synth.initial_state(wl)
    tokens_h, bits_h = st["tokens"].copy(), st["mask_bits"].copy()
    hid_d, w_d, bt_d, bv_d = dev(inp["hidden"]), dev(inp["w"]), dev(bt), dev(bv)
    tok_d, bits_d = dev(tokens_h), dev(bits_h)
    for step in range(3):
        ref = oracle.confidence_unmask(lg, tokens_h, bits_h, wl.S, step, wl.T, wl.gamma, wl.mask_id, tau, kind)
        nm = torch.empty(B, dtype=torch.int32, device="cuda")
        conf = torch.empty(wl.M, device="cuda")
        pred = torch.empty(wl.M, dtype=torch.int32, device="cuda")
        bmd.tt_lmhead_unmask(hid_d, w_d, tok_d, bits_d, nm, step, wl.T, wl.gamma, wl.mask_id, bias_tok=bt_d,
                             bias_val=bv_d, conf_out=conf, pred_out=pred, sampler=kind, temperature=tau)
        torch.cuda.synchronize()
        g = dict(tokens=tok_d.cpu().numpy(), mask_bits=host_bits(bits_d), n_masked=nm.cpu().numpy(),
                 conf=conf.cpu().numpy().reshape(B, wl.S), pred=pred.cpu().numpy().reshape(B, wl.S))
        check_fused_step(wl.S, wl.gamma, step, wl.T, bits_h, g, ref, lambda m: lg[m], wl.mask_id, range(B), kind,
                         temperature=tau)
        tokens_h, bits_h = ref["tokens"], ref["mask_bits"]
        tok_d.copy_(dev(tokens_h))
        bits_d.copy_(dev(bits_h))
