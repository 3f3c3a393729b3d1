"""Pins for the oracle's sampler variants (CPU only): temperature-scaled confidence (the model
card's diffusion example uses temperature 0.1) and the predict-and-noise sampler the wiki page's
"Block-wise generation" section mentions beside confidence unmasking. Closed forms, a library
routine (scipy's softmax) and invariants, not the oracle's own code retyped."""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth


@pytest.mark.parametrize("tau", [0.1, 0.5, 1.0, 2.0])
def test_spike_closed_form_with_temperature(tau):
    V, mask_id, j, delta = 1024, 3, 700, 1.25
    row = np.zeros(V, np.float32)
    row[j] = delta
    conf, a = oracle.reduce_row(row, mask_id, tau)
    e = math.exp(delta / tau)
    assert a == j and conf == pytest.approx(e / (e + V - 2), rel=1e-13)


@pytest.mark.parametrize("tau", [0.1, 0.7, 3.0])
def test_temperature_against_scipy_softmax(tau):
    g = np.random.default_rng(11)
    row = g.normal(size=300).astype(np.float32)
    mask_id = 42
    conf, a = oracle.reduce_row(row, mask_id, tau)
    keep = np.delete(np.arange(300), mask_id)
    p = softmax(row[keep].astype(np.float64) / tau)
    assert conf == pytest.approx(p.max(), rel=1e-13)
    assert a == keep[int(np.argmax(p))]


def test_temperature_keeps_prediction_and_orders_confidence():
    g = np.random.default_rng(12)
    row = g.normal(size=500).astype(np.float32)
    confs = [oracle.reduce_row(row, 3, t)[0] for t in (0.1, 0.3, 1.0, 3.0)]
    preds = {oracle.reduce_row(row, 3, t)[1] for t in (0.1, 0.3, 1.0, 3.0)}
    assert len(preds) == 1
    assert confs == sorted(confs, reverse=True)     # colder = more confident (unique max)
    assert oracle.reduce_row(row, 3, 1e-3)[0] == pytest.approx(1.0, abs=1e-12)


def test_predict_noise_follows_the_linear_schedule():
    """A fully masked block of S = 16 with T = 16 steps keeps floor(16 (15 - t) / 16) = 15 - t
    positions masked after step t: exactly one commit per step, the most confident first."""
    S, T = 16, 16
    conf = np.linspace(0.1, 0.9, S)[::-1]           # position 0 the most confident
    pred = np.arange(100, 100 + S)
    tokens = np.full(S, 3, np.int32)
    bits = (1 << S) - 1
    order = []
    for t in range(T):
        tokens, bits, n, C = oracle.commit_block(conf, pred, tokens, bits, S, t, T, 0.5, "predict_noise")
        assert n == S - 1 - t and len(C) == 1
        order += C
    assert order == list(range(S)) and bits == 0


def test_predict_noise_schedule_with_fewer_steps_and_gamma_ignored():
    S, T = 16, 4          # targets 12, 8, 4, 0
    conf = np.full(S, 0.99)
    tokens = np.full(S, 3, np.int32)
    bits = (1 << S) - 1
    counts = []
    for t in range(T):
        tokens, bits, n, C = oracle.commit_block(conf, np.arange(S), tokens, bits, S, t, T, 0.5, "predict_noise")
        counts.append(n)
        assert C == list(range(4 * t, 4 * t + 4))   # equal confidences: lower positions first
    assert counts == [12, 8, 4, 0]


def test_predict_noise_partial_block_waits_for_the_schedule():
    """Only 5 of 16 positions masked: nothing commits until the target drops below 5."""
    S, T = 16, 16
    conf = np.full(S, 0.5)
    bits = 0b1010100100010000
    tokens = np.where([(bits >> i) & 1 for i in range(S)], 3, 7).astype(np.int32)
    commits = []
    for t in range(T):
        tokens, bits, n, C = oracle.commit_block(conf, np.arange(S), tokens, bits, S, t, T, 0.8, "predict_noise")
        commits.append(len(C))
    assert commits[:11] == [0] * 11 and sum(commits) == 5 and bits == 0


def test_block_sizes_8_32_64_finish_within_t_steps():
    for S in (8, 32, 64):
        wl = synth.workload(0, S=S, B=2, V=256)
        wl.wid = 900 + S
        logits = synth.direct_logits(wl)
        st = synth.initial_state(wl)
        tokens, bits = st["tokens"], st["mask_bits"]
        for t in range(wl.T):
            r = oracle.confidence_unmask(logits, tokens, bits, S, t, wl.T, wl.gamma, wl.mask_id, 0.1)
            tokens, bits = r["tokens"], r["mask_bits"]
        assert np.all(bits == 0) and np.all(tokens != wl.mask_id)
