"""Pins for the oracle's context-tower step over a committed block (CPU only).

Each test checks the oracle against something other than itself: a brute-force per-key
evaluation, torch's scaled-dot-product attention with its causal mask (float64) for the prefix-free
case, closed forms, the causality the wiki page's "Block-wise generation" section implies (the
context tower processes the committed tokens causally), and the append's exact copy."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _inputs(B=2, S=4, Hq=4, Hkv=2, D=8, prefixes=(5, 0), dtype="f32", seed=0):
    wl = synth.workload(0, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, prefixes=list(prefixes), dtype=dtype)
    wl.wid = 300 + seed
    return wl, synth.context_inputs(wl)


def _brute(inp, dtype):
    """Per-key loops with math.fsum / math.exp; new row j visible to position s iff j <= s."""
    q = oracle.decode(inp["q"], dtype)
    kb, vb = oracle.decode(inp["k_blk"], dtype), oracle.decode(inp["v_blk"], dtype)
    kc, vc = oracle.decode(inp["k_ctx"], dtype), oracle.decode(inp["v_ctx"], dtype)
    B, S, Hq, D = q.shape
    G = Hq // kb.shape[2]
    out = np.zeros_like(q)
    for b in range(B):
        a, n = int(inp["ctx_start"][b]), int(inp["ctx_len"][b])
        for s in range(S):
            for h in range(Hq):
                g = h // G
                keys = [kc[g, r] for r in range(a, a + n)] + [kb[b, j, g] for j in range(s + 1)]
                vals = [vc[g, r] for r in range(a, a + n)] + [vb[b, j, g] for j in range(s + 1)]
                z = [inp["scale"] * math.fsum(q[b, s, h, d] * k[d] for d in range(D)) for k in keys]
                mz = max(z)
                e = [math.exp(x - mz) for x in z]
                tot = math.fsum(e)
                for d in range(D):
                    out[b, s, h, d] = math.fsum(e[j] * vals[j][d] for j in range(len(keys))) / tot
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_brute_force_tiny(dtype):
    _, inp = _inputs(dtype=dtype)
    out, _, _, _ = oracle.context_extend(inp, dtype)
    assert np.max(np.abs(out - _brute(inp, dtype))) <= 1e-12


def test_prefix_free_is_torch_causal_sdpa():
    """No cached rows: plain causal self-attention over the new tokens (library routine)."""
    _, inp = _inputs(B=2, S=6, Hq=6, Hkv=2, D=16, prefixes=(0, 0))
    out, _, _, _ = oracle.context_extend(inp, "f32")
    q = torch.from_numpy(oracle.decode(inp["q"], "f32")).permute(0, 2, 1, 3)        # [B][Hq][S][D]
    G = 3
    k = torch.from_numpy(oracle.decode(inp["k_blk"], "f32")).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    v = torch.from_numpy(oracle.decode(inp["v_blk"], "f32")).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=inp["scale"])
    assert np.max(np.abs(out - ref.permute(0, 2, 1, 3).numpy())) <= 1e-12


def test_first_position_without_prefix_returns_its_value():
    _, inp = _inputs(B=1, S=5, prefixes=(0,))
    out, _, _, _ = oracle.context_extend(inp, "f32")
    vb = oracle.decode(inp["v_blk"], "f32")
    for h in range(4):
        assert np.array_equal(out[0, 0, h], vb[0, 0, h // 2])


def test_later_rows_do_not_reach_earlier_positions():
    """Changing new rows j > s leaves position s unchanged; changing row s changes it."""
    _, inp = _inputs(B=2, S=6, prefixes=(3, 9))
    out, _, _, _ = oracle.context_extend(inp, "f32")
    s = 2
    mod = dict(inp)
    mod["k_blk"] = inp["k_blk"].copy()
    mod["v_blk"] = inp["v_blk"].copy()
    mod["k_blk"][:, s + 1:] *= 3.0
    mod["v_blk"][:, s + 1:] -= 1.0
    out2, _, _, _ = oracle.context_extend(mod, "f32")
    assert np.array_equal(out2[:, :s + 1], out[:, :s + 1])
    assert np.max(np.abs(out2[:, s + 1:] - out[:, s + 1:])) > 1e-3
    mod["v_blk"][:, s] += 1.0
    out3, _, _, _ = oracle.context_extend(mod, "f32")
    assert np.max(np.abs(out3[:, s] - out[:, s])) > 1e-3


def test_constant_values_give_that_constant():
    _, inp = _inputs(B=2, S=4, prefixes=(6, 1))
    inp = dict(inp)
    inp["v_ctx"] = np.full_like(inp["v_ctx"], 0.75)
    inp["v_blk"] = np.full_like(inp["v_blk"], 0.75)
    out, _, _, _ = oracle.context_extend(inp, "f32")
    assert np.max(np.abs(out - 0.75)) <= 1e-15


def test_append_copies_rows_and_touches_nothing_else():
    wl, inp = _inputs(B=3, S=4, prefixes=(5, 0, 2), dtype="bf16")
    _, kc, vc, ln = oracle.context_extend(inp, "bf16")
    assert list(ln) == [9, 4, 6]
    changed = np.zeros(kc.shape[1], bool)
    for b in range(3):
        r0 = int(inp["ctx_start"][b] + inp["ctx_len"][b])
        for j in range(4):
            assert np.array_equal(kc[:, r0 + j], inp["k_blk"][b, j])
            assert np.array_equal(vc[:, r0 + j], inp["v_blk"][b, j])
            changed[r0 + j] = True
    assert np.array_equal(kc[:, ~changed], inp["k_ctx"][:, ~changed])
    assert np.array_equal(vc[:, ~changed], inp["v_ctx"][:, ~changed])


def test_layout_reserves_room_after_each_sequence():
    wl, inp = _inputs(B=3, S=4, prefixes=(5, 0, 2))
    assert list(inp["ctx_start"]) == [0, 9, 13] and inp["k_ctx"].shape[1] == 19


def test_last_position_sees_the_whole_block():
    """Position S-1 sees every new row: the same visible set as the denoiser's bidirectional
    block attention, whose own pins are in test_oracle_attention.py."""
    _, inp = _inputs(B=2, S=5, prefixes=(4, 7))
    out, _, _, _ = oracle.context_extend(inp, "f32")
    full = oracle.block_attention(inp, "f32")
    assert np.max(np.abs(out[:, -1] - full[:, -1])) <= 1e-14
    assert np.max(np.abs(out[:, 0] - full[:, 0])) > 1e-3
