"""GPU parity of tt_context_extend (the context tower's causal attention over a committed block,
then the append of its keys/values) against the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL_BF16, ATOL_F32, dev

pytestmark = pytest.mark.gpu

bmd = pytest.importorskip("block_mask_diffusion_amd")


def _run(inp, wl):
    d = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    out = bmd.tt_context_extend(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["ctx_start"],
                                d["ctx_len"], max_prefix=wl.max_prefix, softmax_scale=d["scale"])
    torch.cuda.synchronize()

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
    return (out.float().cpu().numpy().astype(np.float64), host(d["k_ctx"]), host(d["v_ctx"]),
            d["ctx_len"].cpu().numpy())


def _splits_inside_a_block(wl):
    """Whether the launch's key split (256 workgroups at most, 128 keys each at least, a multiple
    of the unit count when there are more workgroups than units, key lists of all (sequence, kv
    head) units end to end) cuts some unit inside its last S keys."""
    U = wl.B * wl.Hkv
    W = max(1, min(256, -(-U * (wl.max_prefix + wl.S) // 128)))
    if W > U:
        W -= W % U
    lens = [p + wl.S for p in wl.prefixes]
    T = wl.Hkv * sum(lens)
    starts, acc = [], 0
    for n in lens:
        for _ in range(wl.Hkv):
            starts.append((acc, n))
            acc += n
    cuts = [w * T // W for w in range(1, W)]
    return any(o + n - wl.S < c < o + n for (o, n) in starts for c in cuts)


def _check(wl, inp=None):
    inp = synth.context_inputs(wl) if inp is None else inp
    got, kc, vc, ln = _run(inp, wl)
    ref, rkc, rvc, rln = oracle.context_extend(inp, wl.dtype)
    tol = ATOL_BF16 if wl.dtype == "bf16" else ATOL_F32
    err = float(np.max(np.abs(got - ref)))
    assert err <= tol, err
    assert np.array_equal(kc, rkc) and np.array_equal(vc, rvc)
    assert np.array_equal(ln, rln)
    return err


@pytest.mark.parametrize("prefixes", [[0], [1], [63], [64], [65], [0, 100, 1000], [777, 5, 130]])
def test_bf16_ragged_prefixes(prefixes):
    wl = synth.workload(1, B=len(prefixes), prefixes=prefixes)
    wl.wid = 600 + sum(prefixes) % 97
    _check(wl)


@pytest.mark.parametrize("S,Hq,Hkv,D,dtype", [(16, 32, 2, 64, "bf16"), (1, 4, 4, 128, "bf16"),
                                              (5, 12, 3, 64, "bf16"), (16, 4, 1, 64, "f32"),
                                              (7, 8, 2, 128, "f32")])
def test_head_layouts(S, Hq, Hkv, D, dtype):
    wl = synth.workload(1, B=2, S=S, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, prefixes=[300, 47])
    wl.wid = 650 + S * Hq + D
    _check(wl)


def test_key_split_cuts_inside_the_block():
    """Pieces of the split that start inside the block leave rows with no visible key (an empty
    partial); the merge must ignore them."""
    found = 0
    for p in range(100, 3000, 7):
        wl = synth.workload(1, B=3, prefixes=[p, 500, 77])
        if _splits_inside_a_block(wl):
            wl.wid = 700 + p % 89
            _check(wl)
            found += 1
        if found == 3:
            break
    assert found == 3


def test_workload_shape_full_prefix():
    """128K-token prefixes (the benchmark's largest shape, one layer): every output row against
    the oracle, every appended row and the lengths exactly."""
    wl = synth.workload(4)
    inp = synth.context_inputs(wl)
    got, kc, vc, ln = _run(inp, wl)
    ref = oracle.context_extend(inp, "bf16")[0]
    err = float(np.max(np.abs(got - ref)))
    assert err <= ATOL_BF16, err
    assert list(ln) == [p + wl.S for p in wl.prefixes]
    for b in range(wl.B):
        r0 = int(inp["ctx_start"][b] + inp["ctx_len"][b])
        assert np.array_equal(kc[:, r0:r0 + wl.S], inp["k_blk"][b].transpose(1, 0, 2))
        assert np.array_equal(vc[:, r0:r0 + wl.S], inp["v_blk"][b].transpose(1, 0, 2))
        assert np.array_equal(kc[:, inp["ctx_start"][b]:r0], inp["k_ctx"][:, inp["ctx_start"][b]:r0])


def test_two_blocks_in_a_row_grow_the_cache():
    """Two committed blocks back to back: the second call sees the first block's rows as prefix."""
    wl = synth.workload(1, B=2, prefixes=[40, 9], S=8, Hq=8, Hkv=2)
    wl.wid = 720
    cap = [p + 2 * wl.S for p in wl.prefixes]
    start = np.array([0, cap[0]], np.int32)
    inp1 = synth.context_inputs(wl)
    # re-lay the cache with room for two blocks per sequence
    R = sum(cap)
    kc = np.zeros((wl.Hkv, R, wl.D), inp1["k_ctx"].dtype)
    vc = np.zeros_like(kc)
    for b in range(2):
        n = wl.prefixes[b]
        a = int(inp1["ctx_start"][b])
        kc[:, start[b]:start[b] + n] = inp1["k_ctx"][:, a:a + n]
        vc[:, start[b]:start[b] + n] = inp1["v_ctx"][:, a:a + n]
    inp1 = dict(inp1, k_ctx=kc, v_ctx=vc, ctx_start=start)
    wl2 = synth.workload(1, B=2, prefixes=[p + wl.S for p in wl.prefixes], S=8, Hq=8, Hkv=2)
    wl2.wid = 721
    nxt = synth.attn_inputs(wl2)
    d = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp1.items()}
    bmd.tt_context_extend(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["ctx_start"], d["ctx_len"],
                          max_prefix=wl.max_prefix, softmax_scale=d["scale"])
    out2 = bmd.tt_context_extend(dev(nxt["q"]), dev(nxt["k_blk"]), dev(nxt["v_blk"]), d["k_ctx"], d["v_ctx"],
                                 d["ctx_start"], d["ctx_len"], max_prefix=wl2.max_prefix, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    _, k1, v1, l1 = oracle.context_extend(inp1, "bf16")
    inp2 = dict(q=nxt["q"], k_blk=nxt["k_blk"], v_blk=nxt["v_blk"], k_ctx=k1, v_ctx=v1, ctx_start=start,
                ctx_len=l1, scale=nxt["scale"])
    ref2, k2, v2, l2 = oracle.context_extend(inp2, "bf16")
    assert float(np.max(np.abs(out2.float().cpu().numpy() - ref2))) <= ATOL_BF16
    assert np.array_equal(d["ctx_len"].cpu().numpy(), l2)
    assert np.array_equal(d["k_ctx"].view(torch.int16).cpu().numpy().view(np.uint16), k2)


def test_deterministic():
    wl = synth.workload(1, B=3, prefixes=[3000, 17, 900])
    wl.wid = 730
    inp = synth.context_inputs(wl)
    a = _run(inp, wl)[0]
    b = _run(inp, wl)[0]
    assert np.array_equal(a, b)


def test_sequences_outside_the_contract_get_no_append():
    """One sequence inside the contract, one with ctx_len above max_prefix, one whose S new rows
    would pass ctx_rows: the attention reads the clamped rows (start within [0, ctx_rows], length
    within [0, min(max_prefix, ctx_rows - start)]); only the first sequence is appended to."""
    wl = synth.workload(1, B=3, prefixes=[100, 60, 40])
    wl.wid = 912
    inp = synth.context_inputs(wl)
    R = inp["k_ctx"].shape[1]
    assert R == 248 and list(inp["ctx_start"]) == [0, 116, 192]
    start = np.array([0, 116, 200], dtype=np.int32)
    length = np.array([100, 120, 40], dtype=np.int32)
    inp["ctx_start"], inp["ctx_len"] = start, length
    got, kc, vc, ln = _run(inp, wl)  # max_prefix = 100
    st = np.clip(start.astype(np.int64), 0, R)
    lc = np.clip(length.astype(np.int64), 0, np.minimum(wl.max_prefix, R - st))
    assert lc.tolist() == [100, 100, 40]
    clamped = dict(inp, ctx_start=st.astype(np.int32), ctx_len=lc.astype(np.int32))
    rows = [(b, s, h) for b in range(wl.B) for s in range(wl.S) for h in range(wl.Hq)]
    ref = oracle.context_extend(clamped, wl.dtype, rows=rows)
    err = max(float(np.max(np.abs(got[r] - ref[r]))) for r in rows)
    assert err <= ATOL_BF16, err
    # the cache as given, with sequence 0's S new rows written after its 100 cached rows
    ekc, evc = np.array(inp["k_ctx"], copy=True), np.array(inp["v_ctx"], copy=True)
    for j in range(wl.S):
        ekc[:, 100 + j] = inp["k_blk"][0, j]
        evc[:, 100 + j] = inp["v_blk"][0, j]
    assert np.array_equal(kc, ekc) and np.array_equal(vc, evc)
    assert ln.tolist() == [116, 120, 40]
