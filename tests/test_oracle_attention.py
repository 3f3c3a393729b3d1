"""Pins for the oracle's block attention (CPU only).

Each test checks the oracle against something other than itself: a brute-force
per-key evaluation, a library routine (torch SDPA in float64) on the special cases
it covers, closed forms, and the symmetries the wiki page's "Architecture" section
implies (bidirectional attention inside the block, context keys before the block)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _inputs(B=2, S=3, Hq=4, Hkv=2, D=8, prefixes=(5, 0), dtype="f32", seed=0):
    wl = synth.workload(0, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, prefixes=list(prefixes), dtype=dtype)
    wl.wid = 100 + seed
    return wl, synth.attn_inputs(wl)


def _brute(inp, dtype):
    """Independent evaluation: explicit per-key loops, math.fsum and math.exp."""
    q = oracle.decode(inp["q"], dtype)
    kb, vb = oracle.decode(inp["k_blk"], dtype), oracle.decode(inp["v_blk"], dtype)
    kc, vc = oracle.decode(inp["k_ctx"], dtype), oracle.decode(inp["v_ctx"], dtype)
    B, S, Hq, D = q.shape
    Hkv = kb.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for s in range(S):
            for h in range(Hq):
                g = h // G
                keys, vals = [], []
                for r in range(int(inp["ctx_start"][b]), int(inp["ctx_start"][b]) + int(inp["ctx_len"][b])):
                    keys.append(kc[g, r]); vals.append(vc[g, r])
                for j in range(S):
                    keys.append(kb[b, j, g]); vals.append(vb[b, j, g])
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
    ref = _brute(inp, dtype)
    got = oracle.block_attention(inp, dtype)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_probabilities_sum_to_one():
    _, inp = _inputs(B=2, S=5, Hq=6, Hkv=3, D=16, prefixes=(7, 2))
    _, probs = oracle.block_attention(inp, "f32", return_probs=True)
    for (b, g), p in probs.items():
        assert p.shape[-1] == int(inp["ctx_len"][b]) + 5
        assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-13)
        assert np.all(p >= 0)


def _sdpa(q, k, v, scale):
    """torch SDPA in float64 on the CPU. q [Hq][Lq][D], k/v [Hq][Lk][D] (heads already repeated)."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()


def test_prefix_zero_is_plain_bidirectional_self_attention():
    _, inp = _inputs(B=2, S=7, Hq=6, Hkv=2, D=16, prefixes=(0, 0), dtype="bf16")
    got = oracle.block_attention(inp, "bf16")
    q = oracle.decode(inp["q"], "bf16")
    k = oracle.decode(inp["k_blk"], "bf16")
    v = oracle.decode(inp["v_blk"], "bf16")
    G = 3
    for b in range(2):
        qh = np.ascontiguousarray(q[b].transpose(1, 0, 2))                     # [Hq][S][D]
        kh = np.repeat(np.ascontiguousarray(k[b].transpose(1, 0, 2)), G, axis=0)  # contiguous groups
        vh = np.repeat(np.ascontiguousarray(v[b].transpose(1, 0, 2)), G, axis=0)
        ref = _sdpa(qh, kh, vh, inp["scale"]).transpose(1, 0, 2)
        assert np.max(np.abs(got[b] - ref)) <= 1e-12


def test_mha_with_prefix_matches_sdpa_over_concatenated_keys():
    _, inp = _inputs(B=2, S=4, Hq=3, Hkv=3, D=8, prefixes=(6, 3))
    got = oracle.block_attention(inp, "f32")
    q = oracle.decode(inp["q"], "f32")
    for b in range(2):
        a, n = int(inp["ctx_start"][b]), int(inp["ctx_len"][b])
        k = np.concatenate([oracle.decode(inp["k_ctx"][:, a:a + n], "f32"),
                            oracle.decode(inp["k_blk"][b].transpose(1, 0, 2), "f32")], axis=1)
        v = np.concatenate([oracle.decode(inp["v_ctx"][:, a:a + n], "f32"),
                            oracle.decode(inp["v_blk"][b].transpose(1, 0, 2), "f32")], axis=1)
        ref = _sdpa(np.ascontiguousarray(q[b].transpose(1, 0, 2)), k, v, inp["scale"]).transpose(1, 0, 2)
        assert np.max(np.abs(got[b] - ref)) <= 1e-12


def test_block_key_permutation_invariance_and_query_equivariance():
    _, inp = _inputs(B=1, S=8, Hq=4, Hkv=2, D=8, prefixes=(5,))
    base = oracle.block_attention(inp, "f32")
    perm = np.random.default_rng(3).permutation(8)
    inp2 = dict(inp)
    inp2["k_blk"] = inp["k_blk"][:, perm]
    inp2["v_blk"] = inp["v_blk"][:, perm]
    assert np.max(np.abs(oracle.block_attention(inp2, "f32") - base)) <= 1e-13
    inp3 = dict(inp)
    inp3["q"] = inp["q"][:, perm]
    assert np.max(np.abs(oracle.block_attention(inp3, "f32") - base[:, perm])) <= 1e-13


def test_closed_forms():
    _, inp = _inputs(B=2, S=4, Hq=4, Hkv=2, D=8, prefixes=(5, 3))
    # every value row equal to c  ->  output c
    c = np.linspace(-1, 1, 8).astype(np.float32)
    i1 = dict(inp, v_ctx=np.broadcast_to(c, inp["v_ctx"].shape).copy(),
              v_blk=np.broadcast_to(c, inp["v_blk"].shape).copy())
    o = oracle.block_attention(i1, "f32")
    assert np.max(np.abs(o - c.astype(np.float64))) <= 1e-14
    # K == 0  ->  uniform weights: output is the mean of all P_b + S value rows
    i2 = dict(inp, k_ctx=np.zeros_like(inp["k_ctx"]), k_blk=np.zeros_like(inp["k_blk"]))
    o = oracle.block_attention(i2, "f32")
    for b in range(2):
        a, n = int(inp["ctx_start"][b]), int(inp["ctx_len"][b])
        for h in range(4):
            g = h // 2
            rows = np.concatenate([inp["v_ctx"][g, a:a + n], inp["v_blk"][b, :, g]]).astype(np.float64)
            assert np.max(np.abs(o[b, :, h] - rows.mean(axis=0))) <= 1e-14
    # a single key (P = 0, S = 1)  ->  output is that value row
    _, i3 = _inputs(B=1, S=1, Hq=2, Hkv=1, D=8, prefixes=(0,))
    o = oracle.block_attention(i3, "f32")
    assert np.array_equal(o[0, 0, 0], i3["v_blk"][0, 0, 0].astype(np.float64))
    assert np.array_equal(o[0, 0, 1], i3["v_blk"][0, 0, 0].astype(np.float64))


def test_packing_offset_does_not_matter():
    """Sequence 1 alone (ctx_start 0) equals sequence 1 packed after sequence 0."""
    _, inp = _inputs(B=2, S=4, Hq=4, Hkv=2, D=8, prefixes=(6, 5))
    both = oracle.block_attention(inp, "f32")
    a, n = int(inp["ctx_start"][1]), int(inp["ctx_len"][1])
    alone = dict(q=inp["q"][1:], k_blk=inp["k_blk"][1:], v_blk=inp["v_blk"][1:],
                 k_ctx=inp["k_ctx"][:, a:a + n], v_ctx=inp["v_ctx"][:, a:a + n],
                 ctx_start=np.array([0], np.int32), ctx_len=np.array([n], np.int32), scale=inp["scale"])
    assert np.max(np.abs(oracle.block_attention(alone, "f32")[0] - both[1])) <= 1e-14


def test_row_subset_matches_full():
    _, inp = _inputs(B=2, S=4, Hq=4, Hkv=2, D=8, prefixes=(6, 5))
    full = oracle.block_attention(inp, "f32")
    rows = [(0, 1, 3), (1, 0, 0), (1, 3, 2)]
    sub = oracle.block_attention(inp, "f32", rows=rows)
    for r in rows:
        assert np.max(np.abs(sub[r] - full[r])) <= 1e-15
