"""The seeded generators: determinism, shapes and the workloads' stated distributions."""
import numpy as np

import oracle
import synth


def test_deterministic_and_shapes():
    wl = synth.workload(0)
    a, b = synth.attn_inputs(wl), synth.attn_inputs(wl)
    for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx"):
        assert np.array_equal(a[k], b[k])
    assert a["q"].shape == (1, 16, 4, 64) and a["q"].dtype == np.float32
    assert a["k_ctx"].shape == (1, 64, 64)
    wl1 = synth.workload(1, V=4096)
    li = synth.lmhead_inputs(wl1)
    assert li["w"].shape == (4096, 2688) and li["w"].dtype == np.uint16
    assert abs(oracle.decode(li["w"][:512], "bf16").std() - 0.02) < 0.001


def test_ragged_prefixes():
    wl = synth.workload(3)
    assert len(wl.prefixes) == 32
    assert min(wl.prefixes) >= 512 and max(wl.prefixes) <= 32768
    assert np.array_equal(wl.ctx_start, np.concatenate([[0], np.cumsum(wl.prefixes)[:-1]]))


def test_partial_initial_state():
    wl = synth.workload(2)
    st = synth.initial_state(wl)
    for b in range(8):
        n = bin(int(st["mask_bits"][b])).count("1")
        if b < 4:
            assert n == 16
        else:
            assert 4 <= 16 - n <= 12
        for i in range(16):
            assert ((int(st["mask_bits"][b]) >> i) & 1) == (st["tokens"][b, i] == 3)


def test_tiny_pass_rate_statistics():
    """Workload 0 draws (N(0,1) noise, one Uniform[0,12] spike per row, V = 1024): the rate of
    rows whose confidence reaches 0.8 is about 0.265 (Monte Carlo estimate); check within 4 sigma."""
    wl = synth.workload(0, B=250)
    logits = synth.direct_logits(wl)
    confs = [oracle.reduce_row(logits[r], 3)[0] for r in range(logits.shape[0])]
    rate = float(np.mean(np.array(confs) >= 0.8))
    sigma = np.sqrt(0.265 * 0.735 / len(confs))
    assert abs(rate - 0.265) <= 4 * sigma
