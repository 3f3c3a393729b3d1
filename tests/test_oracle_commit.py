"""Pins for the oracle's confidence-unmasking commit (CPU only): hand-worked traces,
the special cases gamma > 1 and gamma <= 0, the fixed-logits step count, and the
invariants the wiki page's "Block-wise generation" section states."""
import numpy as np
import pytest

import oracle
import synth
from golden_traces import load


@pytest.mark.parametrize("tr", load(), ids=lambda t: t.name)
def test_hand_worked_trace(tr):
    tokens = np.array([tr.init_tokens], np.int32)
    bits = np.array([tr.init_bits], np.uint64)
    for st in tr.steps:
        r = oracle.confidence_unmask(tr.logits, tokens, bits, tr.S, st["step"], tr.T, tr.gamma, tr.mask_id)
        assert r["committed"][0] == st["commit"]
        assert list(r["tokens"][0]) == st["tokens"]
        assert int(r["mask_bits"][0]) == st["bits"]
        assert int(r["n_masked"][0]) == st["n"]
        tokens, bits = r["tokens"], r["mask_bits"]


def _c0_logits(salt):
    wl = synth.workload(0)
    return wl, synth.direct_logits(wl, salt=salt)


def _run_block(wl, logits, gamma, T=16, tokens=None, bits=None):
    st = synth.initial_state(wl) if tokens is None else dict(tokens=tokens, mask_bits=bits)
    tokens, bits = st["tokens"], st["mask_bits"]
    hist = []
    for step in range(T):
        r = oracle.confidence_unmask(logits, tokens, bits, wl.S, step, T, gamma, wl.mask_id)
        hist.append(r)
        tokens, bits = r["tokens"], r["mask_bits"]
    return hist


@pytest.mark.parametrize("salt", range(3))
def test_gamma_above_one_commits_one_per_step_in_confidence_order(salt):
    wl, logits = _c0_logits(salt)
    hist = _run_block(wl, logits, gamma=1.5)
    conf0 = hist[0]["conf"][0]
    order = sorted(range(16), key=lambda i: (-conf0[i], i))
    for t, r in enumerate(hist):
        assert len(r["committed"][0]) == 1
        assert r["committed"][0][0] == order[t]
        assert int(r["n_masked"][0]) == 15 - t
    assert int(hist[-1]["mask_bits"][0]) == 0


def test_gamma_nonpositive_commits_everything_at_step_zero():
    wl, logits = _c0_logits(7)
    for gamma in (0.0, -1.0):
        r = oracle.confidence_unmask(logits, synth.initial_state(wl)["tokens"],
                                     synth.initial_state(wl)["mask_bits"], 16, 0, 16, gamma, 3)
        assert r["committed"][0] == list(range(16)) and int(r["n_masked"][0]) == 0


@pytest.mark.parametrize("salt", range(6))
def test_fixed_logits_step_count(salt):
    wl, logits = _c0_logits(100 + salt)
    hist = _run_block(wl, logits, gamma=0.8)
    c0 = len([i for i in range(16) if hist[0]["conf"][0][i] >= 0.8])
    steps = sum(1 for r in hist if r["conf"][0].max() >= 0)    # steps that saw >= 1 masked position
    assert steps == (16 if c0 == 0 else 1 + (16 - c0))


@pytest.mark.parametrize("T", [16, 8, 5, 1])
def test_invariants_partial_blocks(T):
    wl = synth.workload(2, B=8, V=1024, H=64)
    logits = synth.direct_logits(wl, noise_std=1.0)
    st = synth.initial_state(wl)
    tokens, bits = st["tokens"], st["mask_bits"]
    prev_n = np.array([bin(int(b)).count("1") for b in bits])
    for step in range(T):
        r = oracle.confidence_unmask(logits, tokens, bits, 16, step, T, 0.8, wl.mask_id)
        for b in range(8):
            for i in range(16):
                was_masked = (int(bits[b]) >> i) & 1
                now_masked = (int(r["mask_bits"][b]) >> i) & 1
                if not was_masked:
                    assert r["tokens"][b, i] == tokens[b, i] and not now_masked
                assert bool(now_masked) == (r["tokens"][b, i] == wl.mask_id)
            n = int(r["n_masked"][b])
            assert n == bin(int(r["mask_bits"][b])).count("1")
            if prev_n[b] > 0:
                assert n < prev_n[b]
            prev_n[b] = n
        tokens, bits = r["tokens"], r["mask_bits"]
    assert np.all(r["n_masked"] == 0)
    assert np.all(tokens != wl.mask_id)


def test_rows_of_committed_positions_are_never_read():
    wl, logits = _c0_logits(11)
    logits = logits.copy()
    st = synth.initial_state(wl)
    bits = np.array([np.uint64(0xFF00)], np.uint64)
    tokens = st["tokens"].copy()
    tokens[0, :8] = np.arange(10, 18)
    logits[:8] = np.nan
    r = oracle.confidence_unmask(logits, tokens, bits, 16, 0, 16, 0.8, 3)
    assert list(r["tokens"][0, :8]) == list(range(10, 18))
    assert np.all(r["conf"][0, :8] == -1.0) and np.all(r["pred"][0, :8] == -1)
