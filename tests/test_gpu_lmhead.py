"""GPU parity of tt_lmhead_logits against the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL_BF16, ATOL_F32, dev

pytestmark = pytest.mark.gpu

bmd = pytest.importorskip("block_mask_diffusion_amd")


def _run(inp):
    out = bmd.tt_lmhead_logits(dev(inp["hidden"]), dev(inp["w"]))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _bound(inp, dtype):
    """fp32 accumulation bound over H terms: |err| <= gamma_H * sum_k |h_k w_k| (+ output rounding)."""
    h = np.abs(oracle.decode(inp["hidden"], dtype))
    w = np.abs(oracle.decode(inp["w"], dtype))
    H = h.shape[1]
    u = 2.0 ** -24
    return (H * u / (1 - H * u)) * (h @ w.T) + 1e-30


@pytest.mark.parametrize("M,H,V,dtype", [(16, 64, 1024, "f32"), (5, 96, 1000, "f32"), (48, 64, 300, "f32"),
                                         (16, 2688, 4096, "bf16"), (48, 96, 1000, "bf16"),
                                         (128, 2688, 2048, "bf16"), (64, 2688, 2304, "bf16"),
                                         (512, 2688, 1024, "bf16"), (100, 288, 777, "bf16"), (1, 32, 256, "bf16"),
                                         (7, 256, 1001, "bf16"), (24, 256, 1000, "bf16"), (65, 128, 513, "bf16"),
                                         (16, 96, 2000, "bf16"), (130, 2688, 700, "bf16"),
                                         # up to 16 rows the vocabulary tile follows V: 64, 128, 256
                                         # rows per workgroup (one GPU's shard of an 8-way split first)
                                         (16, 2688, 16384, "bf16"), (16, 256, 70001, "bf16"),
                                         (9, 128, 131000, "bf16"),
                                         # 17-128 rows: the LDS-staged kernel while V <= 32768 and
                                         # V M <= 2^21; else the GEMM, its 256 x 256 tile while V <= 32768
                                         (40, 256, 32768, "bf16"), (40, 256, 32769, "bf16"),
                                         (64, 2688, 16384, "bf16"), (128, 256, 16384, "bf16"),
                                         (128, 256, 16385, "bf16"), (100, 256, 32769, "bf16"),
                                         # 17-64 rows above V = 32768: the GEMM's 64 x 256 tile with
                                         # its 4-deep ring; ragged vocabulary tails
                                         (33, 128, 65537, "bf16"), (64, 192, 40000, "bf16"),
                                         (17, 64, 40961, "bf16")])
def test_full_compare(M, H, V, dtype):
    wl = synth.workload(1, B=1, H=H, V=V, dtype=dtype)
    wl.B, wl.S = 1, M
    wl.wid = 700 + M + H + V
    inp = synth.lmhead_inputs(wl)
    got = _run(inp)
    ref = oracle.lmhead_logits(inp["hidden"], inp["w"], dtype)
    err = np.abs(got - ref)
    assert float(err.max()) <= (ATOL_BF16 if dtype == "bf16" else ATOL_F32)
    assert np.all(err <= _bound(inp, dtype) + np.abs(ref) * 2.0 ** -24)


def test_one_hot_hidden_reads_weight_columns_exactly():
    wl = synth.workload(1, V=3000, H=256)
    wl.wid = 801
    w = synth.lmhead_inputs(wl)["w"]
    hid = np.zeros((32, 256), np.float32)
    for m in range(32):
        hid[m, (m * 7) % 256] = 1.0
    got = _run(dict(hidden=synth.to_bf16_bits(hid), w=w))
    for m in range(32):
        assert np.array_equal(got[m], oracle.decode(w[:, (m * 7) % 256], "bf16"))


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_workload_full_size(wid):
    """The whole M x 131072 logits matrix of each workload (H = 2688) against the oracle: within
    1e-2 and within the fp32 accumulation bound, entry by entry."""
    wl = synth.workload(wid)
    inp = synth.lmhead_inputs(wl)
    got = _run(inp)
    ref = oracle.lmhead_logits(inp["hidden"], inp["w"], "bf16")
    err = np.abs(got - ref)
    print(f"w{wid}: logits max abs err {float(err.max()):.3e}")
    assert float(err.max()) <= ATOL_BF16
    assert np.all(err <= _bound(inp, "bf16") + np.abs(ref) * 2.0 ** -24)


def test_deterministic():
    wl = synth.workload(1, V=8192)
    wl.wid = 802
    inp = synth.lmhead_inputs(wl)
    h, w = dev(inp["hidden"]), dev(inp["w"])
    a = bmd.tt_lmhead_logits(h, w)
    b = bmd.tt_lmhead_logits(h, w)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
