"""GPU parity of tt_block_attn against the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL_BF16, ATOL_F32, attn_dev

pytestmark = pytest.mark.gpu

bmd = pytest.importorskip("block_mask_diffusion_amd")


def _run(inp_np, wl):
    d = attn_dev(inp_np)
    out = bmd.tt_block_attn(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["ctx_start"],
                            d["ctx_len"], max_prefix=wl.max_prefix, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _wl(wid=1, **kw):
    wl = synth.workload(wid, **kw)
    return wl


def _full_check(wl, layer=0):
    inp = synth.attn_inputs(wl, layer)
    got = _run(inp, wl)
    ref = oracle.block_attention(inp, wl.dtype)
    err = float(np.max(np.abs(got - ref)))
    tol = ATOL_BF16 if wl.dtype == "bf16" else ATOL_F32
    assert err <= tol, err
    return got, ref


def test_tiny_fp32_workload():
    _full_check(synth.workload(0))


@pytest.mark.parametrize("prefixes", [[0], [1], [63], [64], [65], [0, 100, 1000], [777, 5, 130]])
def test_bf16_several_tiles_and_ragged_tails(prefixes):
    wl = _wl(1, B=len(prefixes), prefixes=prefixes)
    wl.wid = 400 + sum(prefixes) % 101
    _full_check(wl)


@pytest.mark.parametrize("S,Hq,Hkv,D,dtype", [(16, 32, 2, 64, "bf16"), (8, 8, 2, 128, "bf16"),
                                              (1, 4, 4, 128, "bf16"), (16, 16, 1, 128, "bf16"),
                                              (5, 12, 3, 64, "bf16"), (16, 4, 1, 64, "f32"),
                                              (16, 8, 2, 128, "f32"), (3, 2, 1, 64, "f32")])
def test_head_layouts(S, Hq, Hkv, D, dtype):
    wl = _wl(1, B=2, S=S, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, prefixes=[300, 47])
    wl.wid = 500 + S * Hq + D
    _full_check(wl)


def test_workload_1_full():
    _full_check(synth.workload(1))


def test_workload_2_full():
    _full_check(synth.workload(2))


def _sampled_check(wl, layer=0, n=48, seed=0):
    inp = synth.attn_inputs(wl, layer)
    got = _run(inp, wl)
    g = np.random.default_rng(seed)
    rows = [(int(g.integers(wl.B)), int(g.integers(wl.S)), int(g.integers(wl.Hq))) for _ in range(n)]
    rows += [(0, 0, 0), (wl.B - 1, wl.S - 1, wl.Hq - 1)]
    ref = oracle.block_attention(inp, wl.dtype, rows=rows)
    err = max(float(np.max(np.abs(got[r] - ref[r]))) for r in rows)
    assert err <= ATOL_BF16, err
    # every output is a convex combination of value rows: bounded by their extremes
    assert np.all(np.isfinite(got))
    vmax = max(float(np.abs(oracle.decode(inp["v_ctx"][:, :4096], "bf16")).max()), 6.0)
    assert float(np.abs(got).max()) <= vmax


def test_workload_3_ragged_full():
    """Every output row of the ragged batch-32 workload (64 units, prefixes 512 to 32768)."""
    _full_check(synth.workload(3))


def test_workload_4_one_layer_full():
    """Every output row of one layer of the batch-4, 131072-token-prefix workload."""
    _full_check(synth.workload(4), layer=5)


def test_workload_4_other_layer_sampled():
    _sampled_check(synth.workload(4), layer=2)


def test_block_key_permutation_invariance():
    wl = _wl(1, B=2, prefixes=[200, 1500])
    wl.wid = 601
    inp = synth.attn_inputs(wl)
    base = _run(inp, wl)
    perm = np.random.default_rng(1).permutation(wl.S)
    inp2 = dict(inp, k_blk=inp["k_blk"][:, perm].copy(), v_blk=inp["v_blk"][:, perm].copy())
    assert float(np.max(np.abs(_run(inp2, wl) - base))) <= 2e-3
    inp3 = dict(inp, q=inp["q"][:, perm].copy())
    assert float(np.max(np.abs(_run(inp3, wl) - base[:, perm]))) <= 2e-3


def test_deterministic():
    wl = synth.workload(3)
    inp = synth.attn_inputs(wl)
    d = attn_dev(inp)
    outs = [bmd.tt_block_attn(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["ctx_start"],
                              d["ctx_len"], max_prefix=wl.max_prefix) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_extreme_scores_exercise_running_max():
    """Q and K scaled by 8 (exact in bf16): scores spread over hundreds of units, so a wrong row
    max (e.g. one wave half not seeing the other's maximum) or a missed rescale overflows the
    exponentials and shows up as inf/NaN or a large error. The softmax is then nearly one-hot and
    outputs approach single value rows; V is halved (exact) so that |o| stays below 4, where the
    bf16 output rounding alone cannot exceed the 1e-2 bound."""
    wl = _wl(1, B=3, prefixes=[700, 1500, 64])
    wl.wid = 610
    inp = synth.attn_inputs(wl)
    for k, f in (("q", 8.0), ("k_blk", 8.0), ("k_ctx", 8.0), ("v_blk", 0.5), ("v_ctx", 0.5)):
        inp[k] = synth.to_bf16_bits(oracle.decode(inp[k], "bf16").astype(np.float32) * f)
    got = _run(inp, wl)
    ref = oracle.block_attention(inp, wl.dtype)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - ref))) <= ATOL_BF16


def test_growing_scores_rescale_at_many_steps():
    """Context keys scaled by a factor that grows from 1 to 8 along the prefix: each row's max
    keeps rising by more than 2^8 in the exponent every few 32-key sub-tiles, so the lazy rescale
    fires at many positions of the pipelined sub-tile loop (all 8 steps of a ring turn) and in
    pieces that straddle units. A rescale applied to the wrong PV product, or skipped, overflows
    or mis-weights the output. V is halved (exact) so |o| stays below 4."""
    wl = _wl(1, B=2, prefixes=[3000, 1100])
    wl.wid = 611
    inp = synth.attn_inputs(wl)
    kc = oracle.decode(inp["k_ctx"], "bf16").astype(np.float32)
    for b in range(wl.B):
        a, n = int(inp["ctx_start"][b]), int(inp["ctx_len"][b])
        kc[:, a:a + n] *= (1.0 + 7.0 * np.arange(n, dtype=np.float32) / n)[None, :, None]
    inp["k_ctx"] = synth.to_bf16_bits(kc)
    for k in ("v_blk", "v_ctx"):
        inp[k] = synth.to_bf16_bits(oracle.decode(inp[k], "bf16").astype(np.float32) * 0.5)
    got = _run(inp, wl)
    ref = oracle.block_attention(inp, wl.dtype)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - ref))) <= ATOL_BF16


def _sweep_cases(n=24, seed=2024):
    """Seeded random shapes: batch 1-5, block size 1-16, grouped heads with S*G <= 256, head_dim
    64 or 128, prefixes from 0 to 3000 (so pieces start and end anywhere in the unrolled loop's
    ring turn, and workgroups take one or several pieces)."""
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        D = int(g.choice([64, 128]))
        Hkv = int(g.choice([1, 2, 3, 4]))
        G = int(g.choice([1, 2, 4, 8, 16]))
        S = int(g.integers(1, 17))
        if S * G > 256:
            continue
        B = int(g.integers(1, 6))
        pref = [int(x) for x in g.integers(0, 3001, size=B)]
        cases.append((B, S, Hkv * G, Hkv, D, pref))
    return cases


@pytest.mark.parametrize("case", _sweep_cases())
def test_random_shape_sweep(case):
    B, S, Hq, Hkv, D, pref = case
    wl = _wl(1, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, prefixes=pref)
    wl.wid = 800 + (sum(pref) + 31 * S + Hq) % 997
    _full_check(wl)


def _clamped(start, length, ctx_rows, max_prefix):
    """The rows the call attends to for lengths outside the caller's contract (include/tt.h):
    start within [0, ctx_rows], then length within [0, min(max_prefix, ctx_rows - start)]."""
    st = np.clip(np.asarray(start, dtype=np.int64), 0, ctx_rows)
    cap = np.minimum(max_prefix, ctx_rows - st)
    ln = np.clip(np.asarray(length, dtype=np.int64), 0, cap)
    return st.astype(np.int32), ln.astype(np.int32)


def test_lengths_outside_the_contract_are_clamped():
    """Every way out of the contract at once, beside one sequence inside it: a length above
    max_prefix, a negative length, a negative start, rows past ctx_rows, a start past ctx_rows.
    The output is the attention over the clamped rows, read within the cache."""
    wl = _wl(1, B=6, prefixes=[200, 50, 120, 80, 30, 64])
    wl.wid = 911
    inp = synth.attn_inputs(wl)
    R = inp["k_ctx"].shape[1]
    assert R == 544
    max_prefix = 150
    start = np.array([0, 200, -40, 500, 600, 480], dtype=np.int32)
    length = np.array([200, -5, 120, 80, 7, 64], dtype=np.int32)
    inp["ctx_start"], inp["ctx_len"] = start, length
    d = attn_dev(inp)
    got = bmd.tt_block_attn(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["ctx_start"],
                            d["ctx_len"], max_prefix=max_prefix, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    st, ln = _clamped(start, length, R, max_prefix)
    assert st.tolist() == [0, 200, 0, 500, 544, 480] and ln.tolist() == [150, 0, 120, 44, 0, 64]
    ref = oracle.block_attention(dict(inp, ctx_start=st, ctx_len=ln), wl.dtype)
    err = float(np.max(np.abs(got - ref)))
    assert err <= ATOL_BF16, err
    # the arrays themselves are inputs only
    assert np.array_equal(d["ctx_start"].cpu().numpy(), start)
    assert np.array_equal(d["ctx_len"].cpu().numpy(), length)


def _nan_workspace(nbytes):
    return torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device="cuda")  # fp32 NaN bytes


@pytest.mark.parametrize("B,prefixes,max_prefix", [(1, [0], 4096), (1, [100], 131072), (2, [0, 5], 8192),
                                                   (2, [3, 0], 131072), (2, [40, 300], 65536)])
def test_short_sequences_against_a_large_max_prefix(B, prefixes, max_prefix):
    """max_prefix sizes the launch (its workgroup count), the lengths on the device may be far
    shorter: most workgroups then own no keys and write no partial. The merge must read only the
    partials that were written; a workspace filled with NaN shows any stale read."""
    wl = _wl(1, B=B, prefixes=prefixes)
    wl.wid = 1300 + sum(prefixes) + max_prefix % 97
    inp = synth.attn_inputs(wl)
    # the cache holds 64 rows more than the sequences use (never attended: a cache sized for
    # later blocks), so it is not empty even when every length is 0
    spare = synth._store(synth._normal(synth.rng(wl.wid, synth.T_SPARE), (wl.Hkv, 64, wl.D)), wl.dtype)
    inp["k_ctx"] = np.concatenate([inp["k_ctx"], spare], axis=1)
    inp["v_ctx"] = np.concatenate([inp["v_ctx"], spare[:, ::-1]], axis=1)
    d = attn_dev(inp)
    n = bmd.workspace_bytes("tt_block_attn", B=B, S=wl.S, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                            ctx_rows=inp["k_ctx"].shape[1], max_prefix=max_prefix)
    out = bmd.tt_block_attn(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["ctx_start"], d["ctx_len"],
                            max_prefix=max_prefix, softmax_scale=d["scale"], workspace=_nan_workspace(n))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.block_attention(inp, wl.dtype)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - ref))) <= ATOL_BF16


@pytest.mark.parametrize("B,prefixes,max_prefix", [(1, [0], 4096), (2, [0, 5], 8192), (2, [40, 300], 16384)])
def test_context_extend_short_sequences_against_a_large_max_prefix(B, prefixes, max_prefix):
    """The same for the context tower's step: a cache with room for max_prefix + S rows, short
    sequences in it, a NaN-filled workspace."""
    wl = _wl(1, B=B, prefixes=prefixes)
    wl.wid = 1350 + sum(prefixes)
    inp = synth.context_inputs(wl)
    R = max_prefix + wl.S + inp["k_ctx"].shape[1]
    pad = ((0, 0), (0, R - inp["k_ctx"].shape[1]), (0, 0))
    inp["k_ctx"] = np.pad(inp["k_ctx"], pad)
    inp["v_ctx"] = np.pad(inp["v_ctx"], pad)
    d = attn_dev(inp)
    n = bmd.workspace_bytes("tt_block_attn", B=B, S=wl.S, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, ctx_rows=R,
                            max_prefix=max_prefix)
    out = bmd.tt_context_extend(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["ctx_start"],
                                d["ctx_len"], max_prefix=max_prefix, softmax_scale=d["scale"],
                                workspace=_nan_workspace(n))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref, kc, vc, ln = oracle.context_extend(inp, wl.dtype)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - ref))) <= ATOL_BF16
    assert np.array_equal(d["ctx_len"].cpu().numpy(), ln)
    assert np.array_equal(d["k_ctx"].view(torch.int16).cpu().numpy().view(np.uint16), kc)
    assert np.array_equal(d["v_ctx"].view(torch.int16).cpu().numpy().view(np.uint16), vc)
