"""GPU parity of tt_lmhead_unmask (LM head + confidence unmask with the vocabulary reduction in
the LM-head epilogue; the logits are never stored) against the oracle: fp64 LM head, the
per-row logit bias added to the one entry, then the oracle's confidence unmask. Inputs are the
seeded synth draws only. Tolerances are those of gpu_util.check_fused_step."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_fused_step, dev, host_bits

pytestmark = pytest.mark.gpu

bmd = pytest.importorskip("block_mask_diffusion_amd")


def _wl(B, S, H, V, mask_id=3, wid=1, salt=0, partial=False):
    wl = synth.workload(wid, B=B, S=S, H=H, V=V, mask_id=mask_id, partial_init=partial)
    wl.wid = 1000 + 7 * B + 3 * S + H + V % 1009 + salt
    return wl


def _bias(wl, use_bias=True):
    if not use_bias:
        return None, None
    sp = synth.spikes(wl)
    return sp["tok"].astype(np.int32), sp["val"]


def _oracle_logits(inp, bt, bv, rows=None):
    h = inp["hidden"] if rows is None else inp["hidden"][rows]
    lg = oracle.lmhead_logits(h, inp["w"], "bf16")
    if bt is not None:
        r = np.arange(lg.shape[0]) if rows is None else np.asarray(rows)
        lg[np.arange(lg.shape[0]), bt[r]] += bv[r].astype(np.float64)
    return lg


def _fused(hid_d, w_d, bt_d, bv_d, tok_d, bits_d, B, S, step, T, gamma, mask_id):
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    conf = torch.empty(B * S, dtype=torch.float32, device="cuda")
    pred = torch.empty(B * S, dtype=torch.int32, device="cuda")
    bmd.tt_lmhead_unmask(hid_d, w_d, tok_d, bits_d, nm, step, T, gamma, mask_id, bias_tok=bt_d, bias_val=bv_d,
                         conf_out=conf, pred_out=pred)
    torch.cuda.synchronize()
    return dict(tokens=tok_d.cpu().numpy(), mask_bits=host_bits(bits_d), n_masked=nm.cpu().numpy(),
                conf=conf.cpu().numpy().reshape(B, S), pred=pred.cpu().numpy().reshape(B, S))


def _steps(wl, steps, use_bias=True, gamma=None, inp=None):
    """Run `steps` fused steps against the oracle from the initial state; both sides continue
    from the oracle's state after each step. Returns (exempt blocks, rel conf errors, state)."""
    gamma = wl.gamma if gamma is None else gamma
    inp = synth.lmhead_inputs(wl) if inp is None else inp
    bt, bv = _bias(wl, use_bias)
    lg = _oracle_logits(inp, bt, bv)
    st = synth.initial_state(wl)
    tokens_h, bits_h = st["tokens"].copy(), st["mask_bits"].copy()
    hid_d, w_d = dev(inp["hidden"]), dev(inp["w"])
    bt_d = None if bt is None else dev(bt)
    bv_d = None if bv is None else dev(bv)
    tok_d, bits_d = dev(tokens_h), dev(bits_h)
    exempt, rel = 0, []
    for step in range(steps):
        ref = oracle.confidence_unmask(lg, tokens_h, bits_h, wl.S, step, wl.T, gamma, wl.mask_id)
        g = _fused(hid_d, w_d, bt_d, bv_d, tok_d, bits_d, wl.B, wl.S, step, wl.T, gamma, wl.mask_id)
        e, r = check_fused_step(wl.S, gamma, step, wl.T, bits_h, g, ref, lambda m: lg[m], wl.mask_id,
                                range(wl.B))
        exempt += e
        rel += r
        tokens_h, bits_h = ref["tokens"], ref["mask_bits"]
        tok_d.copy_(dev(tokens_h))
        bits_d.copy_(dev(bits_h))
    return exempt, np.array(rel), tokens_h, bits_h


# shapes: each hidden-row bucket (<= 16 rows, <= 64, <= 128, > 128), ragged vocabularies
# (not a multiple of any column block), several k-stages, S from 1 to 64
@pytest.mark.parametrize("B,S,H,V,mask_id", [
    (1, 16, 256, 4099, 3), (1, 7, 128, 1000, 999), (3, 16, 128, 1000, 0), (4, 16, 192, 2050, 64),
    (5, 16, 192, 3001, 127), (12, 13, 128, 2050, 128), (1, 64, 64, 300, 3), (2, 1, 64, 2, 1),
    (3, 33, 64, 777, 5), (9, 16, 320, 1537, 3), (2, 16, 256, 16384, 3),
    # 17-64 rows above V = 32768: the GEMM's 64 x 256 tile (64-column records), ragged tails, the
    # mask id in the last block
    (3, 16, 128, 40000, 7), (2, 13, 192, 33001, 33000),
])
def test_fused_against_oracle(B, S, H, V, mask_id):
    wl = _wl(B, S, H, V, mask_id)
    exempt, rel, _, _ = _steps(wl, 2)
    print(f"fused B={B} S={S} H={H} V={V}: exempt blocks {exempt}, conf rel err max {rel.max():.2e}")


@pytest.mark.parametrize("use_bias", [False, True])
def test_fused_full_block(use_bias):
    wl = _wl(2, 16, 128, 2000, salt=int(use_bias))
    _, _, tokens, bits = _steps(wl, wl.T, use_bias=use_bias)
    assert np.all(bits == 0) and np.all(tokens != wl.mask_id)


@pytest.mark.parametrize("gamma", [2.0, 0.0, float("-inf")])
def test_fused_gamma_extremes(gamma):
    wl = _wl(2, 16, 64, 1024, salt=11)
    _steps(wl, 3, gamma=gamma)


def test_fused_partly_committed_blocks_and_nan_rows():
    """Committed positions are never reduced: their hidden rows may hold NaN."""
    wl = _wl(4, 16, 128, 1500, partial=True)
    inp = synth.lmhead_inputs(wl)
    st = synth.initial_state(wl)
    bt, bv = _bias(wl)
    lg = _oracle_logits(inp, bt, bv)
    hid = inp["hidden"].copy()
    for b in range(wl.B):
        for i in range(wl.S):
            if not (int(st["mask_bits"][b]) >> i) & 1:
                hid[b * wl.S + i] = 0x7FC0     # bf16 quiet NaN
    ref = oracle.confidence_unmask(lg, st["tokens"], st["mask_bits"], wl.S, 0, wl.T, wl.gamma, wl.mask_id)
    g = _fused(dev(hid), dev(inp["w"]), dev(bt), dev(bv), dev(st["tokens"]), dev(st["mask_bits"]), wl.B, wl.S,
               0, wl.T, wl.gamma, wl.mask_id)
    check_fused_step(wl.S, wl.gamma, 0, wl.T, st["mask_bits"], g, ref, lambda m: lg[m], wl.mask_id, range(wl.B))
    assert np.all(np.isfinite(g["conf"]))


def test_bias_on_mask_id_and_outside_vocab_adds_nothing_visible():
    wl = _wl(1, 16, 64, 1000, mask_id=3, salt=5)
    inp = synth.lmhead_inputs(wl)
    bt = np.full(16, 3, np.int32)
    bt[8:] = [-1, 1000, 5000, -7, 2 ** 31 - 1, 1000, 999, 0]
    bv = np.full(16, 50.0, np.float32)
    lg = _oracle_logits(inp, None, None)
    lg_b = lg.copy()
    for m in range(16):
        if 0 <= bt[m] < wl.V:
            lg_b[m, bt[m]] += 50.0
    st = synth.initial_state(wl)
    ref = oracle.confidence_unmask(lg_b, st["tokens"], st["mask_bits"], 16, 0, wl.T, wl.gamma, wl.mask_id)
    g = _fused(dev(inp["hidden"]), dev(inp["w"]), dev(bt), dev(bv), dev(st["tokens"]), dev(st["mask_bits"]), 1,
               16, 0, wl.T, wl.gamma, wl.mask_id)
    check_fused_step(16, wl.gamma, 0, wl.T, st["mask_bits"], g, ref, lambda m: lg_b[m], wl.mask_id, [0])
    assert np.all(g["pred"][0][:8] != 3)
    assert g["pred"][0][14] == 999 and g["pred"][0][15] == 0


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_workload_full_size_sampled(wid):
    """Full-size LM head (H 2688, V 131072) at each workload's row count, in the launch the
    benchmark times; the oracle checks two whole blocks (every row of them) one row at a time."""
    wl = synth.workload(wid)
    inp = synth.lmhead_inputs(wl)
    sp = synth.spikes(wl)
    bt, bv = sp["tok"].astype(np.int32), sp["val"]
    st = synth.initial_state(wl)
    g = _fused(dev(inp["hidden"]), dev(inp["w"]), dev(bt), dev(bv), dev(st["tokens"]), dev(st["mask_bits"]),
               wl.B, wl.S, 0, wl.T, wl.gamma, wl.mask_id)
    blocks = sorted({0, wl.B - 1})
    rows = [b * wl.S + i for b in blocks for i in range(wl.S)]
    lg_rows = _oracle_logits(inp, bt, bv, rows)
    lg = {r: lg_rows[j] for j, r in enumerate(rows)}
    # the oracle's unmask over just these blocks (rows of other blocks are never read)
    ref_conf = np.full((wl.B, wl.S), -1.0)
    ref_pred = np.full((wl.B, wl.S), -1, np.int64)
    ref_tok = st["tokens"].copy()
    ref_bits = st["mask_bits"].copy()
    ref_nm = np.zeros(wl.B, np.int32)
    for b in blocks:
        bits = int(st["mask_bits"][b])
        for i in range(wl.S):
            if (bits >> i) & 1:
                ref_conf[b, i], ref_pred[b, i] = oracle.reduce_row(lg[b * wl.S + i], wl.mask_id)
        t, nb, nm, _ = oracle.commit_block(ref_conf[b], ref_pred[b], st["tokens"][b], bits, wl.S, 0, wl.T, wl.gamma)
        ref_tok[b], ref_bits[b], ref_nm[b] = t, np.uint64(nb), nm
    ref = dict(tokens=ref_tok, mask_bits=ref_bits, n_masked=ref_nm, conf=ref_conf, pred=ref_pred)
    exempt, rel = check_fused_step(wl.S, wl.gamma, 0, wl.T, st["mask_bits"], g, ref, lambda m: lg[m], wl.mask_id,
                                   blocks)
    print(f"fused w{wid}: exempt blocks {exempt}, conf rel err max {max(rel):.2e}")


def test_fused_equals_two_call_path():
    """Same fp32 accumulators as tt_lmhead_logits: predictions identical, confidences equal to
    fp32 summation-order rounding, identical commits (HIP against HIP, beside the oracle tests)."""
    for B in (1, 4, 8, 12):
        wl = _wl(B, 16, 192, 3000, salt=B)
        inp = synth.lmhead_inputs(wl)
        bt, bv = _bias(wl)
        st = synth.initial_state(wl)
        hid_d, w_d = dev(inp["hidden"]), dev(inp["w"])
        g = _fused(hid_d, w_d, dev(bt), dev(bv), dev(st["tokens"]), dev(st["mask_bits"]), B, 16, 0, wl.T,
                   wl.gamma, wl.mask_id)
        logits = bmd.tt_lmhead_logits(hid_d, w_d)
        logits[torch.arange(wl.M, device="cuda"), dev(bt).long()] += dev(bv)
        tok_d, bits_d = dev(st["tokens"]), dev(st["mask_bits"])
        nm = torch.empty(B, dtype=torch.int32, device="cuda")
        conf = torch.empty(wl.M, dtype=torch.float32, device="cuda")
        pred = torch.empty(wl.M, dtype=torch.int32, device="cuda")
        bmd.tt_confidence_unmask(logits, tok_d, bits_d, nm, 0, wl.T, wl.gamma, wl.mask_id, conf, pred)
        torch.cuda.synchronize()
        assert np.array_equal(pred.cpu().numpy().reshape(B, 16), g["pred"])
        c2 = conf.cpu().numpy().reshape(B, 16)
        assert np.all(np.abs(c2 - g["conf"]) <= 1e-6 * np.abs(c2) + 1e-12)
        near = np.abs(c2 - wl.gamma) <= 1e-5
        for b in range(B):
            if not near[b].any():
                assert np.array_equal(tok_d.cpu().numpy()[b], g["tokens"][b])


def test_fused_deterministic():
    wl = _wl(8, 16, 256, 5000, salt=3)
    inp = synth.lmhead_inputs(wl)
    bt, bv = _bias(wl)
    outs = []
    for _ in range(2):
        st = synth.initial_state(wl)
        outs.append(_fused(dev(inp["hidden"]), dev(inp["w"]), dev(bt), dev(bv), dev(st["tokens"]),
                           dev(st["mask_bits"]), wl.B, wl.S, 0, wl.T, wl.gamma, wl.mask_id))
    for k in ("tokens", "mask_bits", "n_masked", "pred"):
        assert np.array_equal(outs[0][k], outs[1][k])
    assert np.array_equal(outs[0]["conf"].view(np.uint32), outs[1]["conf"].view(np.uint32))


def test_fp32_inputs_are_unsupported():
    wl = _wl(1, 16, 64, 256)
    h = torch.zeros((16, 64), dtype=torch.float32, device="cuda")
    w = torch.zeros((256, 64), dtype=torch.float32, device="cuda")
    st = synth.initial_state(wl)
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(bmd.TTError):
        bmd.tt_lmhead_unmask(h, w, dev(st["tokens"]), dev(st["mask_bits"]), nm, 0, 16, 0.8, 3)


def test_fused_gemm_masked_rows_only_with_nan_committed_rows():
    """More than 128 rows: the product runs over the still-masked rows only (compacted in the
    kernel); committed rows' hidden states may hold NaN. Several steps, so the masked count
    crosses the 256-row tile boundary."""
    wl = _wl(28, 16, 128, 1500, partial=True, salt=21)
    inp = synth.lmhead_inputs(wl)
    st = synth.initial_state(wl)
    bt, bv = _bias(wl)
    lg = _oracle_logits(inp, bt, bv)
    tokens_h, bits_h = st["tokens"].copy(), st["mask_bits"].copy()
    hid = inp["hidden"].copy()
    for b in range(wl.B):
        for i in range(wl.S):
            if not (int(bits_h[b]) >> i) & 1:
                hid[b * wl.S + i] = 0x7FC0     # bf16 quiet NaN in rows committed before step 0
    hid_d, w_d, bt_d, bv_d = dev(hid), dev(inp["w"]), dev(bt), dev(bv)
    tok_d, bits_d = dev(tokens_h), dev(bits_h)
    counts = []
    for step in range(6):
        counts.append(sum(bin(int(x)).count("1") for x in bits_h))
        ref = oracle.confidence_unmask(lg, tokens_h, bits_h, wl.S, step, wl.T, wl.gamma, wl.mask_id)
        g = _fused(hid_d, w_d, bt_d, bv_d, tok_d, bits_d, wl.B, wl.S, step, wl.T, wl.gamma, wl.mask_id)
        check_fused_step(wl.S, wl.gamma, step, wl.T, bits_h, g, ref, lambda m: lg[m], wl.mask_id, range(wl.B))
        tokens_h, bits_h = ref["tokens"], ref["mask_bits"]
        tok_d.copy_(dev(tokens_h))
        bits_d.copy_(dev(bits_h))
    assert counts[0] > 256 and min(counts) < 256


def test_fused_gemm_nothing_masked():
    wl = _wl(18, 16, 64, 700, salt=22)
    inp = synth.lmhead_inputs(wl)
    tokens = np.arange(wl.M, dtype=np.int32).reshape(wl.B, wl.S) % wl.V
    tokens[tokens == wl.mask_id] = 0
    bits = np.zeros(wl.B, np.uint64)
    g = _fused(dev(inp["hidden"]), dev(inp["w"]), None, None, dev(tokens), dev(bits), wl.B, wl.S, 0, wl.T,
               wl.gamma, wl.mask_id)
    assert np.array_equal(g["tokens"], tokens) and np.all(g["mask_bits"] == 0) and np.all(g["n_masked"] == 0)
    assert np.all(g["conf"] == -1.0) and np.all(g["pred"] == -1)


def test_fused_gemm_full_block_to_completion():
    wl = _wl(20, 16, 64, 900, salt=23)
    _, _, tokens, bits = _steps(wl, wl.T)
    assert np.all(bits == 0) and np.all(tokens != wl.mask_id)


@pytest.mark.parametrize("B,S", [(20, 16), (3, 16), (10, 13), (9, 64)])
def test_mask_bits_above_S_are_ignored(B, S):
    """Bits at or above S name no position. Both unmask calls ignore them (no row is read or
    reduced for them, no record lands outside the workspace) and store them back unchanged; every
    other output equals the call on the same word without them. B = 20, S = 16 runs the fused
    call's masked-row compaction (more than 128 rows), where a stray bit of the last block would
    otherwise name a row past the end."""
    wl = _wl(B, S, 128, 1500, partial=True, salt=31 + S)
    inp = synth.lmhead_inputs(wl)
    st = synth.initial_state(wl)
    bt, bv = _bias(wl)
    valid = (1 << S) - 1 if S < 64 else (1 << 64) - 1
    g = np.random.default_rng(S)
    stray = np.array([int(g.integers(0, 1 << 62)) & ~valid for _ in range(B)], dtype=np.uint64)
    hid_d, w_d, bt_d, bv_d = dev(inp["hidden"]), dev(inp["w"]), dev(bt), dev(bv)
    need = bmd.workspace_bytes("tt_lmhead_unmask", B=B, S=S, H=128, V=wl.V)
    counters = -(-64 * (B + B * S) // 256) * 256
    guard = 1 << 16
    res = []
    for bits in (st["mask_bits"], st["mask_bits"] | stray):
        ws = torch.full((need + guard,), 0xAB, dtype=torch.uint8, device="cuda")
        ws[:counters] = 0   # the arrival counters start at zero; the rest of the workspace is scratch
        tok_d, bits_d = dev(st["tokens"]), dev(bits)
        nm = torch.empty(B, dtype=torch.int32, device="cuda")
        conf = torch.empty(wl.M, dtype=torch.float32, device="cuda")
        pred = torch.empty(wl.M, dtype=torch.int32, device="cuda")
        bmd.tt_lmhead_unmask(hid_d, w_d, tok_d, bits_d, nm, 0, wl.T, wl.gamma, wl.mask_id, bias_tok=bt_d,
                             bias_val=bv_d, conf_out=conf, pred_out=pred, workspace=ws)
        # the three-call path on the same word
        logits = bmd.tt_lmhead_logits(hid_d, w_d)
        tok3, bits3 = dev(st["tokens"]), dev(bits)
        nm3 = torch.empty(B, dtype=torch.int32, device="cuda")
        bmd.tt_confidence_unmask(logits, tok3, bits3, nm3, 0, wl.T, wl.gamma, wl.mask_id)
        torch.cuda.synchronize()
        assert torch.all(ws[need:] == 0xAB), "a record landed past the workspace"
        assert torch.all(ws[:counters] == 0), "the arrival counters were not left at zero"
        res.append(dict(tok=tok_d.cpu().numpy(), bits=host_bits(bits_d), nm=nm.cpu().numpy(),
                        conf=conf.cpu().numpy(), pred=pred.cpu().numpy(), tok3=tok3.cpu().numpy(),
                        bits3=host_bits(bits3), nm3=nm3.cpu().numpy()))
    lo, hi = res
    for k in ("tok", "nm", "pred", "tok3", "nm3"):
        assert np.array_equal(lo[k], hi[k]), k
    assert np.array_equal(lo["conf"].view(np.uint32), hi["conf"].view(np.uint32))
    assert np.array_equal(hi["bits"], lo["bits"] | stray)
    assert np.array_equal(hi["bits3"], lo["bits3"] | stray)
