"""Pins for the oracle's LM head, input decoding and vocabulary reduction (CPU only)."""
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth


# ----------------------------------------------------------------- bf16 storage

def test_bf16_round_and_decode_known_values():
    x = np.array([1.0, -2.0, 1.0 + 2 ** -7, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.140625, 65280.0],
                 dtype=np.float32)
    bits = synth.to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6)
    assert list(bits) == [0x3F80, 0xC000, 0x3F81, 0x3F80, 0x3F82, 0x4049, 0x477F]
    assert list(oracle.decode(bits, "bf16")) == [1.0, -2.0, 1.0 + 2 ** -7, 1.0, 1.0 + 2 ** -6, 3.140625, 65280.0]


# ----------------------------------------------------------------- LM head

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lmhead_against_fsum(dtype):
    g = np.random.default_rng(1)
    h = g.standard_normal((3, 5)).astype(np.float32)
    w = g.standard_normal((7, 5)).astype(np.float32)
    if dtype == "bf16":
        h, w = synth.to_bf16_bits(h), synth.to_bf16_bits(w)
    got = oracle.lmhead_logits(h, w, dtype)
    hd, wd = oracle.decode(h, dtype), oracle.decode(w, dtype)
    for m in range(3):
        for v in range(7):
            assert abs(got[m, v] - math.fsum(hd[m, k] * wd[v, k] for k in range(5))) <= 1e-14


def test_lmhead_one_hot_hidden_reads_a_weight_column_exactly():
    g = np.random.default_rng(2)
    w = synth.to_bf16_bits(g.standard_normal((11, 6)).astype(np.float32))
    for k in range(6):
        h = np.zeros((1, 6), np.float32)
        h[0, k] = 1.0
        got = oracle.lmhead_logits(synth.to_bf16_bits(h), w, "bf16")[0]
        assert np.array_equal(got, oracle.decode(w[:, k], "bf16"))


def test_lmhead_entries_match_full_product():
    wl = synth.workload(1, B=1, H=64, V=300)
    wl.wid = 201
    inp = synth.lmhead_inputs(wl)
    full = oracle.lmhead_logits(inp["hidden"], inp["w"], "bf16")
    pairs = [(0, 0), (3, 299), (15, 17)]
    ent = oracle.lmhead_entries(inp["hidden"], inp["w"], "bf16", pairs)
    for (m, v), e in zip(pairs, ent):
        assert abs(full[m, v] - e) <= 1e-12


# ----------------------------------------------------------------- reduction

@pytest.mark.parametrize("mask_id", [0, 3, 9])
def test_all_equal_row(mask_id):
    V = 10
    row = np.full(V, 0.37, np.float32)
    conf, a = oracle.reduce_row(row, mask_id)
    assert conf == pytest.approx(1.0 / (V - 1), abs=1e-15)
    assert a == (1 if mask_id == 0 else 0)


@pytest.mark.parametrize("delta", [0.5, 3.0, 11.5])
def test_single_spike_closed_form(delta):
    V, mask_id, j = 1024, 3, 700
    row = np.zeros(V, np.float32)
    row[j] = delta
    conf, a = oracle.reduce_row(row, mask_id)
    e = math.exp(float(np.float32(delta)))
    assert a == j
    assert conf == pytest.approx(e / (e + V - 2), rel=1e-14)


def test_two_equal_maxima_pick_lower_id():
    row = np.zeros(64, np.float32)
    row[40] = row[17] = 2.0
    conf, a = oracle.reduce_row(row, 3)
    assert a == 17
    assert conf <= 0.5
    e = math.exp(2.0)
    assert conf == pytest.approx(e / (2 * e + 64 - 3), rel=1e-14)


def test_spike_on_mask_is_never_returned():
    row = np.zeros(32, np.float32)
    row[3] = 50.0
    conf, a = oracle.reduce_row(row, 3)
    assert a == 0 and conf == pytest.approx(1.0 / 31, rel=1e-14)


def test_against_scipy_softmax_with_mask_column_removed():
    g = np.random.default_rng(5)
    for mask_id in (0, 3, 511):
        for _ in range(20):
            row = (g.standard_normal(512) * 3).astype(np.float32)
            conf, a = oracle.reduce_row(row, mask_id)
            keep = np.delete(row.astype(np.float64), mask_id)
            p = scipy.special.softmax(keep)
            i = int(np.argmax(p))
            assert conf == pytest.approx(float(p[i]), rel=1e-13)
            assert a == (i + 1 if i >= mask_id else i)
            sm = oracle.masked_softmax(row, mask_id)
            assert sm[mask_id] == 0.0
            assert sm.sum() == pytest.approx(1.0, abs=1e-13)
            assert float(sm.max()) == pytest.approx(conf, rel=1e-13)
