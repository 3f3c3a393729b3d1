"""The C-ABI library on the CPU: it loads, exports every symbol include/tt.h declares, and its
host-side validation and workspace queries behave as documented. Nothing here launches a
kernel: every call below returns before any HIP work (an error, or a size query)."""
import ctypes
import os
import re

import pytest

from block_mask_diffusion_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p(4096)  # non-null placeholder: never dereferenced by the paths tested here


def _declared():
    src = open(os.path.join(ROOT, "include", "tt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.tt_abi_version() >> 16 == 1


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert _lib.status_string(code).startswith("TT_")
    assert _lib.status_string(7) == "unknown status"


def _attn(**kw):
    a = dict(q=P, kb=P, vb=P, kc=P, vc=P, cs=P, cl=P, out=P, B=1, S=16, Hq=32, Hkv=2, D=128,
             ctx_rows=2048, max_prefix=2048, scale=0.088, dtype=_lib.TT_BF16)
    a.update(kw)
    n = ctypes.c_size_t(0)
    st = _lib.load().tt_block_attn(a["q"], a["kb"], a["vb"], a["kc"], a["vc"], a["cs"], a["cl"], a["out"],
                                   a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["ctx_rows"],
                                   a["max_prefix"], a["scale"], a["dtype"], None, ctypes.byref(n), None)
    return st, n.value


def test_attn_workspace_query_and_size():
    st, n = _attn()
    assert st == 0
    # 2 units, 4128 keys -> ceil(4128/128) = 33 workgroups, rounded down to a multiple of the unit
    # count: 32; slots = 32 + 2, R = 256 rows (whole 32-row tiles), D = 128
    # fp32 normalised partials + (m, l) as two fp32 per row
    slots, R, D = 34, 256, 128
    expect = -(-(slots * R * D * 4) // 256) * 256 + -(-(slots * R * 8) // 256) * 256
    assert n == expect
    st, n4 = _attn(B=4, max_prefix=131072, ctx_rows=4 * 131072)
    assert st == 0 and n4 == -(-((256 + 8) * R * D * 4) // 256) * 256 + -(-((256 + 8) * R * 8) // 256) * 256
    st, nf = _attn(dtype=_lib.TT_F32)
    assert st == 0 and nf == n


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(cs=None), -1), (dict(kc=None), -1),
    (dict(B=0), -1), (dict(S=0), -1), (dict(Hq=33), -1), (dict(Hkv=0), -1), (dict(max_prefix=-1), -1),
    (dict(scale=float("nan")), -1), (dict(scale=0.0), -1), (dict(scale=float("inf")), -1),
    (dict(ctx_rows=-1), -1),
    (dict(D=96), -2), (dict(D=256), -2), (dict(dtype=5), -2), (dict(S=17), -2), (dict(B=1025), -2),
])
def test_attn_argument_errors(kw, code):
    assert _attn(**kw)[0] == code


def test_attn_null_context_allowed_without_prefix():
    assert _attn(kc=None, vc=None, max_prefix=0, ctx_rows=0)[0] == 0


def test_attn_workspace_too_small():
    n = ctypes.c_size_t(100)
    st = _lib.load().tt_block_attn(P, P, P, P, P, P, P, P, 1, 16, 32, 2, 128, 2048, 2048, 0.088,
                                   _lib.TT_BF16, P, ctypes.byref(n), None)
    assert st == _lib.TT_ERR_WORKSPACE


def _lm(**kw):
    a = dict(h=P, w=P, out=P, M=16, H=2688, V=131072, dtype=_lib.TT_BF16)
    a.update(kw)
    return _lib.load().tt_lmhead_logits(a["h"], a["w"], a["out"], a["M"], a["H"], a["V"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), -1), (dict(w=None), -1), (dict(out=None), -1), (dict(M=0), -1), (dict(H=-32), -1),
    (dict(V=0), -1), (dict(H=2680), -2), (dict(dtype=3), -2), (dict(h=ctypes.c_void_p(4098)), -1),
])
def test_lmhead_argument_errors(kw, code):
    assert _lm(**kw) == code


def _um(ws=None, nbytes=0, **kw):
    a = dict(lg=P, tok=P, bits=P, nm=P, B=1, S=16, V=131072, step=0, T=16, gamma=0.8, mask_id=3)
    a.update(kw)
    n = ctypes.c_size_t(nbytes)
    st = _lib.load().tt_confidence_unmask(a["lg"], a["tok"], a["bits"], a["nm"], None, None, a["B"], a["S"],
                                          a["V"], a["step"], a["T"], a["gamma"], a["mask_id"], ws,
                                          ctypes.byref(n), None)
    return st, n.value


def _counters(B, S=16):
    """Arrival counters of the B blocks and B*S rows, 64 bytes apart, rounded up to 256 bytes."""
    return -(-64 * (B + B * S) // 256) * 256


def test_unmask_workspace_query():
    # counters, then one 16-byte record per (row, range of 4096-entry chunks) when a row is split
    # (into up to ceil(V / 4096) ranges, so that rows x ranges reaches 1024), then one per row
    st, n = _um()
    assert st == 0 and n == _counters(1) + 16 * 32 * 16 + 16 * 16        # 16 rows x 32 ranges
    st, n = _um(B=32, V=1000)
    assert st == 0 and n == _counters(32) + 512 * 16                     # one chunk: no split
    st, n = _um(B=65, S=1, V=4097)
    assert st == 0 and n == _counters(65, 1) + 65 * 2 * 16 + 65 * 16     # 65 rows x 2 ranges
    st, n = _um(B=8, V=131072)
    assert st == 0 and n == _counters(8) + 128 * 8 * 16 + 128 * 16       # 8 ranges of 4 chunks
    st, n = _um(B=32, V=131072)
    assert st == 0 and n == _counters(32) + 512 * 2 * 16 + 512 * 16      # 2 ranges of 16 chunks
    st, n = _um(B=200, V=131072)
    assert st == 0 and n == _counters(200) + 3200 * 16                   # 3200 rows >= 1024: no split
    assert _um(ws=P, nbytes=10)[0] == _lib.TT_ERR_WORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(lg=None), -1), (dict(tok=None), -1), (dict(bits=None), -1), (dict(nm=None), -1),
    (dict(B=0), -1), (dict(S=0), -1), (dict(V=1), -1), (dict(mask_id=-1), -1), (dict(mask_id=131072), -1),
    (dict(T=0), -1), (dict(step=16), -1), (dict(step=-1), -1), (dict(gamma=float("nan")), -1),
    (dict(S=65), -2), (dict(V=2**31 - 4096, mask_id=3), -2),
])
def test_unmask_argument_errors(kw, code):
    assert _um(**kw)[0] == code


def test_unmasking_workspaces_must_be_256_byte_aligned():
    # the arrival counters at a workspace's start need 256-byte alignment; rejected before any launch
    odd = ctypes.c_void_p(4096 + 16)
    for call in (_um, _fu):
        need = call()[1]
        assert call(ws=odd, nbytes=need + 256)[0] == _lib.TT_ERR_ARG
    assert _lib.load().tt_abi_version() == (1 << 16) | 2


def test_unmask_any_gamma_is_legal():
    for g in (float("inf"), float("-inf"), 2.0, 0.0, -1.0):
        assert _um(gamma=g)[0] == 0


def _fu(ws=None, nbytes=0, **kw):
    a = dict(h=P, w=P, bt=None, bv=None, tok=P, bits=P, nm=P, B=1, S=16, H=2688, V=131072, step=0, T=16,
             gamma=0.8, mask_id=3, dtype=_lib.TT_BF16)
    a.update(kw)
    n = ctypes.c_size_t(nbytes)
    sm = _lib.Sampler(a.get("kind", 0), a["gamma"], a.get("temp", 1.0))
    st = _lib.load().tt_lmhead_unmask(a["h"], a["w"], a["bt"], a["bv"], a["tok"], a["bits"], a["nm"], None, None,
                                      a["B"], a["S"], a["H"], a["V"], a["step"], a["T"], ctypes.byref(sm),
                                      a["mask_id"], a["dtype"], ws, ctypes.byref(n), None)
    return st, n.value


def test_fused_workspace_query():
    # the arrival counters; records per row: 64 columns each up to 64 rows (the LDS-staged kernel
    # to 16 rows, then the GEMM's 64 x 256 tile), 128 beyond; plus one per row
    for B, cols in ((1, 64), (2, 64), (4, 64), (5, 128), (32, 128), (65, 128)):
        M = 16 * B
        st, n = _fu(B=B)
        assert st == 0 and n == _counters(B) + M * (131072 // cols) * 16 + M * 16, (B, n)
    # small vocabularies: the LDS-staged kernel's tile is 64 VT rows with 16 VT columns per
    # record, VT the widest of 4, 2, 1 whose grid (vocabulary tiles x 16-row blocks) reaches 512;
    # up to 128 rows it runs when V <= 32768 and V * rows <= 2^21
    st, n = _fu(V=1000)
    assert st == 0 and n == _counters(1) + 16 * 63 * 16 + 16 * 16      # VT = 1: ceil(1000 / 16) = 63 records per row
    st, n = _fu(B=4, V=16384)
    assert st == 0 and n == _counters(4) + 64 * 512 * 16 + 64 * 16     # VT = 2 (128 x 4 = 512 workgroups): 32 columns
    st, n = _fu(B=8, V=16384)
    assert st == 0 and n == _counters(8) + 128 * 256 * 16 + 128 * 16   # VT = 4 (64 x 8 = 512 workgroups): 64 columns
    st, n = _fu(B=8, V=16385)
    assert st == 0 and n == _counters(8) + 128 * 129 * 16 + 128 * 16   # V * rows above 2^21: the GEMM kernel, 128 columns
    st, n = _fu(B=9, V=16384)
    assert st == 0 and n == _counters(9) + 144 * 128 * 16 + 144 * 16   # 144 rows: the GEMM kernel
    assert _fu(ws=P, nbytes=10)[0] == _lib.TT_ERR_WORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), -1), (dict(w=None), -1), (dict(tok=None), -1), (dict(bits=None), -1), (dict(nm=None), -1),
    (dict(bt=P), -1), (dict(bv=P), -1), (dict(B=0), -1), (dict(S=0), -1), (dict(H=0), -1), (dict(V=1), -1),
    (dict(mask_id=131072), -1), (dict(step=16), -1), (dict(gamma=float("nan")), -1),
    (dict(dtype=_lib.TT_F32), -2), (dict(dtype=7), -2), (dict(H=2656), -2), (dict(S=65), -2),
    (dict(temp=0.0), -1), (dict(temp=-1.0), -1), (dict(temp=float("inf")), -1), (dict(kind=2), -2),
])
def test_fused_argument_errors(kw, code):
    assert _fu(**kw)[0] == code


def test_fused_bias_pair_accepted():
    assert _fu(bt=P, bv=P)[0] == 0


def _ce(ws=None, nbytes=0, **kw):
    a = dict(q=P, kn=P, vn=P, kc=P, vc=P, cs=P, cl=P, out=P, B=1, S=16, Hq=32, Hkv=2, D=128,
             ctx_rows=2048 + 16, max_prefix=2048, scale=0.088, dtype=_lib.TT_BF16)
    a.update(kw)
    n = ctypes.c_size_t(nbytes)
    st = _lib.load().tt_context_extend(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["cs"], a["cl"], a["out"],
                                       a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["ctx_rows"], a["max_prefix"],
                                       a["scale"], a["dtype"], ws, ctypes.byref(n), None)
    return st, n.value


def test_context_extend_workspace_matches_block_attention():
    st, n = _ce()
    st2, n2 = _attn(ctx_rows=2048 + 16)
    assert st == 0 and st2 == 0 and n == n2 > 0
    assert _ce(ws=P, nbytes=10)[0] == _lib.TT_ERR_WORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kn=None), -1), (dict(kc=None, max_prefix=0), -1), (dict(vc=None, max_prefix=0), -1),
    (dict(cl=None), -1), (dict(B=0), -1), (dict(Hq=33), -1), (dict(scale=float("nan")), -1),
    (dict(ctx_rows=2048 + 15), -1), (dict(D=96), -2), (dict(S=17), -2), (dict(dtype=4), -2),
])
def test_context_extend_argument_errors(kw, code):
    assert _ce(**kw)[0] == code


def _us(ws=None, nbytes=0, sampler=True, **kw):
    a = dict(lg=P, tok=P, bits=P, nm=P, B=1, S=16, V=131072, step=0, T=16, mask_id=3, kind=0, gamma=0.8, temp=1.0)
    a.update(kw)
    n = ctypes.c_size_t(nbytes)
    sm = _lib.Sampler(a["kind"], a["gamma"], a["temp"])
    st = _lib.load().tt_unmask_sample(a["lg"], a["tok"], a["bits"], a["nm"], None, None, a["B"], a["S"], a["V"],
                                      a["step"], a["T"], ctypes.byref(sm) if sampler else None, a["mask_id"], ws,
                                      ctypes.byref(n), None)
    return st, n.value


def test_unmask_sample_workspace_equals_confidence_unmask():
    for kind, temp in ((0, 1.0), (1, 0.1), (0, 2.5)):
        st, n = _us(kind=kind, temp=temp)
        assert st == 0 and n == _um()[1]


@pytest.mark.parametrize("kw,code", [
    (dict(sampler=False), -1), (dict(temp=0.0), -1), (dict(temp=float("nan")), -1), (dict(gamma=float("nan")), -1),
    (dict(kind=-1), -2), (dict(kind=7), -2), (dict(lg=None), -1), (dict(S=65), -2), (dict(step=16), -1),
])
def test_unmask_sample_argument_errors(kw, code):
    assert _us(**kw)[0] == code
