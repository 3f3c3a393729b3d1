"""Pin of the oracle's step composition (denoise_step) against the hand-worked block runs of
tests/golden/denoise_trace.txt: one-hot hidden rows make every logits row a known column of W,
spikes are placed by hand, and value rows are constant per layer, so every confidence, prediction,
commit and attention output has a closed form worked out without code.

A spike on the wrong row, a dropped or reordered attention layer, a transposed LM-head product,
the wrong step index (the floor's k) or the wrong threshold test each changes at least one line
of the traces or one closed-form value checked here."""
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "denoise_trace.txt")

B, S, H, V, MASK = 2, 4, 4, 8, 3
# hidden row m is one-hot at COL[m]; SPIKES[m] = (token, value)
COL = [0, 1, 2, 3, 2, 0, 1, 0]
SPIKES = [(2, 5.0), (5, 0.5), (6, 1.0), (3, 4.0), (0, 0.25), (4, 7.0), (5, 3.0), (7, 2.0)]
PRED = [2, 5, 6, 7, 1, 4, 5, 7]
E = math.exp
CONF = [E(5) / (E(5) + 6), E(2.5) / (E(2.5) + 6), E(4) / (E(4) + E(3) + 5), E(1) / (E(1) + 6),
        E(3) / (2 * E(3) + E(0.25) + 4), E(7) / (E(7) + 6), E(5) / (E(5) + 6), E(2) / (E(2) + 6)]
LAYER_C = [0.5, -2.0]


def _w():
    w = np.zeros((V, H), np.float32)
    w[5, 1] = 2.0
    w[1, 2] = w[6, 2] = 3.0
    w[3, 3] = 9.0
    w[7, 3] = 1.0
    return w


def _hidden():
    h = np.zeros((B * S, H), np.float32)
    h[np.arange(B * S), COL] = 1.0
    return h


def _layers():
    """Two attention layers, fp32, Hq = 2, Hkv = 1, D = 4, prefixes 3 and 0; every value row of
    layer l equals LAYER_C[l]."""
    g = np.random.default_rng(7)
    out = []
    for c in LAYER_C:
        rows = 3
        out.append(dict(q=g.standard_normal((B, S, 2, 4)).astype(np.float32),
                        k_blk=g.standard_normal((B, S, 1, 4)).astype(np.float32),
                        v_blk=np.full((B, S, 1, 4), c, np.float32),
                        k_ctx=g.standard_normal((1, rows, 4)).astype(np.float32),
                        v_ctx=np.full((1, rows, 4), c, np.float32),
                        ctx_start=np.array([0, 3], np.int32), ctx_len=np.array([3, 0], np.int32),
                        scale=0.5))
    return out


def _parse():
    scen, cur = {}, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        t = line.split()
        if t[0] == "scenario":
            cur = dict(T=int(t[3]), gamma=float(t[5]), steps={})
            scen[t[1]] = cur
        elif t[0] == "step":
            step, b = int(t[1]), int(t[3])
            commit = [int(x) for x in t[5].split(",")]
            tokens = [int(x) for x in t[7:7 + S]]
            bits, n = int(t[7 + S + 1]), int(t[7 + S + 3])
            cur["steps"][(step, b)] = (commit, tokens, bits, n)
        elif t[0] == "end":
            cur = None
    return scen


def _run(name):
    sc = _parse()[name]
    layers, hid, w = _layers(), _hidden(), _w()
    tok = np.array([s[0] for s in SPIKES], np.int64)
    val = np.array([s[1] for s in SPIKES], np.float32)
    tokens = np.full((B, S), MASK, np.int32)
    bits = np.full(B, (1 << S) - 1, np.uint64)
    for step in range(sc["T"]):
        r = oracle.denoise_step(layers, hid, w, "f32", tok, val, tokens, bits, S, step, sc["T"], sc["gamma"], MASK)
        # attention: one output per layer, in order, each the layer's constant
        assert len(r["attn"]) == len(LAYER_C)
        for o, c in zip(r["attn"], LAYER_C):
            assert o.shape == (B, S, 2, 4)
            assert np.max(np.abs(o - c)) <= 1e-12
        # LM head + spikes: row m is column COL[m] of W plus its spike, exactly
        want = w[:, COL].T.astype(np.float64)
        want[np.arange(B * S), tok] += val
        assert np.array_equal(r["logits"], want)
        for b in range(B):
            commit, t_exp, b_exp, n_exp = sc["steps"][(step, b)]
            assert r["committed"][b] == commit, (name, step, b)
            assert r["tokens"][b].tolist() == t_exp, (name, step, b)
            assert int(r["mask_bits"][b]) == b_exp, (name, step, b)
            assert int(r["n_masked"][b]) == n_exp, (name, step, b)
            for i in range(S):
                if (int(bits[b]) >> i) & 1:
                    assert int(r["pred"][b, i]) == PRED[b * S + i]
                    assert abs(float(r["conf"][b, i]) - CONF[b * S + i]) <= 1e-12
                else:
                    assert float(r["conf"][b, i]) == -1.0 and int(r["pred"][b, i]) == -1
        tokens, bits = r["tokens"], r["mask_bits"]
    assert np.all(bits == 0)
    return tokens


def test_scenario_threshold_and_floor_of_two():
    tokens = _run("one")
    assert tokens.tolist() == [[2, 5, 6, 7], [1, 4, 5, 7]]


def test_scenario_floor_only_descending_confidence():
    tokens = _run("two")
    assert tokens.tolist() == [[2, 5, 6, 7], [1, 4, 5, 7]]


def test_trace_file_is_consistent():
    """Each line of the traces follows from the one before it: commits clear exactly their bits,
    write their hand-derived predictions, and n counts the bits left."""
    for sc in _parse().values():
        for b in range(B):
            tokens, bits = [MASK] * S, (1 << S) - 1
            for step in range(sc["T"]):
                commit, t_exp, b_exp, n_exp = sc["steps"][(step, b)]
                for i in commit:
                    assert (bits >> i) & 1
                    tokens[i] = PRED[b * S + i]
                    bits &= ~(1 << i)
                assert tokens == t_exp and bits == b_exp and bin(bits).count("1") == n_exp
