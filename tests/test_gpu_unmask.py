"""GPU parity of tt_confidence_unmask against the oracle (stage-wise: both sides read the same
fp32 logits, drawn by synth, never produced by the HIP path)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from golden_traces import load as load_traces
from gpu_util import check_commit_step, dev, host_bits

pytestmark = pytest.mark.gpu

bmd = pytest.importorskip("block_mask_diffusion_amd")


def _gpu_step(logits_d, tokens_d, bits_d, S, step, T, gamma, mask_id):
    B = tokens_d.shape[0]
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    conf = torch.empty(B * S, dtype=torch.float32, device="cuda")
    pred = torch.empty(B * S, dtype=torch.int32, device="cuda")
    bmd.tt_confidence_unmask(logits_d, tokens_d, bits_d, nm, step, T, gamma, mask_id, conf, pred)
    torch.cuda.synchronize()
    return dict(tokens=tokens_d.cpu().numpy(), mask_bits=host_bits(bits_d), n_masked=nm.cpu().numpy(),
                conf=conf.cpu().numpy().reshape(B, S), pred=pred.cpu().numpy().reshape(B, S))


@pytest.mark.parametrize("tr", load_traces(), ids=lambda t: t.name)
def test_hand_worked_traces_bit_exact(tr):
    logits = dev(tr.logits)
    tokens = dev(np.array([tr.init_tokens], np.int32))
    bits = dev(np.array([tr.init_bits], np.uint64))
    for st in tr.steps:
        before = int(host_bits(bits)[0])
        g = _gpu_step(logits, tokens, bits, tr.S, st["step"], tr.T, tr.gamma, tr.mask_id)
        assert [i for i in range(tr.S) if (before >> i) & 1 and not (int(g["mask_bits"][0]) >> i) & 1] == st["commit"]
        assert list(g["tokens"][0]) == st["tokens"]
        assert int(g["mask_bits"][0]) == st["bits"] and int(g["n_masked"][0]) == st["n"]


def _run_and_compare(wl, logits_np, steps, gamma=None, state=None):
    gamma = wl.gamma if gamma is None else gamma
    st = synth.initial_state(wl) if state is None else state
    tokens_h, bits_h = st["tokens"].copy(), st["mask_bits"].copy()
    logits_d = dev(logits_np)
    tokens_d, bits_d = dev(tokens_h), dev(bits_h)
    exempt = 0
    for step in range(steps):
        ref = oracle.confidence_unmask(logits_np, tokens_h, bits_h, wl.S, step, wl.T, gamma, wl.mask_id)
        g = _gpu_step(logits_d, tokens_d, bits_d, wl.S, step, wl.T, gamma, wl.mask_id)
        exempt += check_commit_step(wl.S, gamma, step, wl.T, bits_h, tokens_h, g, ref)
        # both sides continue from the oracle's state (the GPU's equals it unless exempt)
        tokens_h, bits_h = ref["tokens"], ref["mask_bits"]
        tokens_d.copy_(dev(tokens_h))
        bits_d.copy_(dev(bits_h))
    return exempt, tokens_h, bits_h


@pytest.mark.parametrize("salt", range(3))
def test_tiny_workload_full_block(salt):
    wl = synth.workload(0)
    logits = synth.direct_logits(wl, salt=salt)
    _, tokens, bits = _run_and_compare(wl, logits, wl.T)
    assert int(bits[0]) == 0 and np.all(tokens != wl.mask_id)


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_full_vocab_workloads_stagewise(wid):
    wl = synth.workload(wid)
    logits = synth.direct_logits(wl)
    _run_and_compare(wl, logits, 3)


@pytest.mark.parametrize("V,mask_id,S,B", [(2, 0, 16, 1), (2, 1, 1, 3), (1001, 1000, 64, 2), (4099, 0, 7, 5),
                                           (8192, 4096, 33, 2), (131071, 3, 16, 2),
                                           # one row of one position in 32 ranges; 64-position
                                           # blocks in 8 ranges of 2 chunks
                                           (131072, 131071, 1, 1), (65536, 7, 64, 2)])
def test_odd_shapes(V, mask_id, S, B):
    wl = synth.workload(0, V=V, mask_id=mask_id, S=S, B=B)
    wl.wid = 300 + V % 97
    logits = synth.direct_logits(wl, noise_std=1.0)
    _run_and_compare(wl, logits, 4)


@pytest.mark.parametrize("B,S,V,partial", [(64, 16, 20000, False), (70, 16, 36867, True), (33, 31, 4097, True)])
def test_one_workgroup_per_row(B, S, V, partial):
    """From 1024 rows on, one workgroup streams a whole row: its whole chunks two at a time with
    the next chunk's loads in flight (odd and even chunk counts), then the ragged last chunk, and
    there is no row ticket. V = 36867 is odd (the scalar-load kernel); partly committed blocks
    leave some rows unread; 1023 rows still split each row in two (one whole chunk, one ragged)."""
    wl = synth.workload(0, B=B, S=S, V=V, mask_id=V // 3, partial_init=partial)
    wl.wid = 400 + B
    logits = synth.direct_logits(wl, noise_std=1.0)
    _run_and_compare(wl, logits, 2)


@pytest.mark.parametrize("gamma", [2.0, float("inf"), 0.0, -1.0])
def test_gamma_extremes(gamma):
    wl = synth.workload(0)
    logits = synth.direct_logits(wl, salt=9)
    _, _, bits = _run_and_compare(wl, logits, wl.T, gamma=gamma)
    assert int(bits[0]) == 0


def test_committed_rows_are_not_read_and_clean_blocks_unchanged():
    wl = synth.workload(0, B=3)
    logits = synth.direct_logits(wl, salt=4)
    logits[16:32] = np.nan              # block 1: fully committed, rows full of NaN
    logits[32:40] = np.nan              # block 2: positions 0..7 committed
    tokens = np.full((3, 16), 3, np.int32)
    tokens[1] = np.arange(100, 116)
    tokens[2, :8] = np.arange(200, 208)
    bits = np.array([0xFFFF, 0, 0xFF00], np.uint64)
    g = _gpu_step(dev(logits), dev(tokens), dev(bits), 16, 0, 16, 0.8, 3)
    assert list(g["tokens"][1]) == list(range(100, 116)) and int(g["mask_bits"][1]) == 0
    assert int(g["n_masked"][1]) == 0
    assert list(g["tokens"][2][:8]) == list(range(200, 208))
    assert np.all(g["conf"][1] == -1.0) and np.all(g["pred"][2][:8] == -1)


def test_deterministic():
    wl = synth.workload(3)
    logits = dev(synth.direct_logits(wl))
    outs = []
    for _ in range(2):
        st = synth.initial_state(wl)
        outs.append(_gpu_step(logits, dev(st["tokens"]), dev(st["mask_bits"]), 16, 0, 16, 0.8, 3))
    for k in ("tokens", "mask_bits", "n_masked", "pred"):
        assert np.array_equal(outs[0][k], outs[1][k])
    assert np.array_equal(outs[0]["conf"].view(np.uint32), outs[1]["conf"].view(np.uint32))


@pytest.mark.parametrize("B,S,V", [(3, 16, 131072), (70, 13, 9000)])
def test_one_workspace_across_a_block(B, S, V):
    """One caller workspace serves every step of a block: the arrival counters at its start are
    zero before the first call and are left zero by each call, so every step equals the same step
    on a fresh zero-filled workspace. B = 3 splits each row into 16 ranges of 2 chunks (row and
    block tickets); B = 70 splits its 910 rows of 3 chunks (the last one ragged) into 2 ranges."""
    wl = synth.workload(1, B=B, S=S, V=V, partial_init=True)
    wl.wid = 1700 + B
    logits = dev(synth.direct_logits(wl))
    st = synth.initial_state(wl)
    need = bmd.workspace_bytes("tt_confidence_unmask", B=B, S=S, V=V)
    counters = -(-64 * (B + B * S) // 256) * 256
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    tok_a, bits_a = dev(st["tokens"]), dev(st["mask_bits"])
    tok_b, bits_b = dev(st["tokens"]), dev(st["mask_bits"])
    for step in range(wl.T):
        nm_a = torch.empty(B, dtype=torch.int32, device="cuda")
        nm_b = torch.empty(B, dtype=torch.int32, device="cuda")
        bmd.tt_confidence_unmask(logits, tok_a, bits_a, nm_a, step, wl.T, wl.gamma, wl.mask_id, workspace=ws)
        bmd.tt_confidence_unmask(logits, tok_b, bits_b, nm_b, step, wl.T, wl.gamma, wl.mask_id)
        torch.cuda.synchronize()
        assert torch.all(ws[:counters] == 0), step
        assert torch.equal(tok_a, tok_b) and torch.equal(bits_a, bits_b) and torch.equal(nm_a, nm_b), step
    assert np.all(host_bits(bits_a) == 0)
