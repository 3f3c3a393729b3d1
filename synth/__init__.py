"""Seeded synthetic inputs for the TwoTower denoiser block step.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
bench. It holds no arithmetic of the method: only random draws, the rounding of
those draws to bf16 storage, and the shape bookkeeping of the five workloads.
Nothing here computes attention, logits, confidences or commit decisions.

Every tensor is drawn from numpy's PCG64 seeded with
``SeedSequence([0, workload_id, tensor_id, layer])`` in float32, then (for bf16
workloads) rounded to bf16 with round-to-nearest-even and handed out as raw
``uint16`` bit patterns, so both sides consume bit-identical inputs.

Workloads (the denoiser operating point of the wiki page "Nemotron-Labs-TwoTower",
section "Block-wise generation": block size S=16, up to 16 steps per block,
gamma=0.8; mask token id 3 from the MLX port's configuration table; contexts up
to 128K tokens from the same wiki page's "Release history and artifacts"):

  0  tiny fp32: B=1, prefix 64, Hq=4, Hkv=1, D=64; logits 16x1024 given directly
  1  bf16 B=1, prefix 2048, Hq=32, Hkv=2, D=128, LM head 2688 x 131072
  2  bf16 B=8, prefix 8192 each; blocks 0..3 fully masked, 4..7 partly committed
  3  bf16 ragged B=32, prefixes UniformInt[512, 32768]
  4  bf16 B=4, prefix 131072 each, six attention layers with separate caches
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# tensor ids for the seed sequence
T_Q, T_KBLK, T_VBLK, T_KCTX, T_VCTX = 1, 2, 3, 4, 5
T_HIDDEN, T_W, T_SPIKE_TOK, T_SPIKE_VAL, T_LOGIT_NOISE = 6, 7, 8, 9, 10
T_LENS, T_MASK_INIT, T_MASK_TOK, T_PERM = 11, 12, 13, 14
T_SPARE = 15  # filler of the cache rows reserved for appends


@dataclass
class Workload:
    """Shapes and sampler parameters of one synthetic workload."""
    wid: int
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    prefixes: List[int]
    H: int
    V: int
    layers: int
    dtype: str                 # "f32" or "bf16"
    gamma: float = 0.8
    T: int = 16
    mask_id: int = 3
    w_std: float = 0.02
    spike_hi: float = 12.0
    partial_init: bool = False  # half the blocks start partly committed
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def M(self) -> int:
        return self.B * self.S

    @property
    def ctx_rows(self) -> int:
        return int(sum(self.prefixes))

    @property
    def max_prefix(self) -> int:
        return int(max(self.prefixes)) if self.prefixes else 0

    @property
    def ctx_start(self) -> np.ndarray:
        p = np.asarray(self.prefixes, dtype=np.int64)
        return (np.cumsum(p) - p).astype(np.int32)

    @property
    def ctx_len(self) -> np.ndarray:
        return np.asarray(self.prefixes, dtype=np.int32)


def rng(wid: int, tensor_id: int, layer: int = 0, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, wid, tensor_id, layer, salt])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to bf16 (round to nearest, ties to even); return uint16 bits.

    Inputs are finite by construction (normal / uniform draws)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def workload(wid: int, **over) -> Workload:
    """The five workloads, by id. Keyword overrides build reduced variants
    (same distributions, smaller shapes) for tests that the oracle must finish quickly."""
    if wid == 0:
        wl = Workload(0, "tiny-f32", B=1, S=16, Hq=4, Hkv=1, D=64, prefixes=[64],
                      H=64, V=1024, layers=1, dtype="f32")
    elif wid == 1:
        wl = Workload(1, "b1-p2048", B=1, S=16, Hq=32, Hkv=2, D=128, prefixes=[2048],
                      H=2688, V=131072, layers=1, dtype="bf16")
    elif wid == 2:
        wl = Workload(2, "b8-p8192-partial", B=8, S=16, Hq=32, Hkv=2, D=128, prefixes=[8192] * 8,
                      H=2688, V=131072, layers=1, dtype="bf16", partial_init=True)
    elif wid == 3:
        g = rng(3, T_LENS)
        pre = [int(v) for v in g.integers(512, 32768, size=32, endpoint=True)]
        wl = Workload(3, "b32-ragged", B=32, S=16, Hq=32, Hkv=2, D=128, prefixes=pre,
                      H=2688, V=131072, layers=1, dtype="bf16")
    elif wid == 4:
        wl = Workload(4, "b4-p131072-6layer", B=4, S=16, Hq=32, Hkv=2, D=128, prefixes=[131072] * 4,
                      H=2688, V=131072, layers=6, dtype="bf16")
    else:
        raise ValueError(f"unknown workload {wid}")
    for k, v in over.items():
        if not hasattr(wl, k):
            raise ValueError(f"unknown workload field {k}")
        setattr(wl, k, v)
    if "B" in over and "prefixes" not in over:
        wl.prefixes = (wl.prefixes * wl.B)[: wl.B]
    return wl


def attn_inputs(wl: Workload, layer: int = 0) -> dict:
    """Q [B][S][Hq][D], K_blk/V_blk [B][S][Hkv][D], K_ctx/V_ctx [Hkv][ctx_rows][D]
    (sequences packed back to back, ctx_start = exclusive prefix sum), all N(0,1)."""
    B, S, Hq, Hkv, D = wl.B, wl.S, wl.Hq, wl.Hkv, wl.D
    R = wl.ctx_rows
    w = wl.wid
    return dict(
        q=_store(_normal(rng(w, T_Q, layer), (B, S, Hq, D)), wl.dtype),
        k_blk=_store(_normal(rng(w, T_KBLK, layer), (B, S, Hkv, D)), wl.dtype),
        v_blk=_store(_normal(rng(w, T_VBLK, layer), (B, S, Hkv, D)), wl.dtype),
        k_ctx=_store(_normal(rng(w, T_KCTX, layer), (Hkv, R, D)), wl.dtype),
        v_ctx=_store(_normal(rng(w, T_VCTX, layer), (Hkv, R, D)), wl.dtype),
        ctx_start=wl.ctx_start,
        ctx_len=wl.ctx_len,
        scale=float(1.0 / np.sqrt(wl.D)),
    )


def context_inputs(wl: Workload, layer: int = 0) -> dict:
    """Inputs of the context tower's step over a committed block: q / k_blk / v_blk as in
    attn_inputs (here the new tokens' queries, keys and values) and a cache laid out with room
    for S more rows per sequence: sequence b owns rows [start_b, start_b + prefix_b + S), the
    first prefix_b of them cached, the last S filled with N(0,1) filler to be overwritten."""
    B, S, Hq, Hkv, D = wl.B, wl.S, wl.Hq, wl.Hkv, wl.D
    p = np.asarray(wl.prefixes, dtype=np.int64)
    cap = p + S
    start = (np.cumsum(cap) - cap).astype(np.int32)
    R = int(cap.sum())
    base = attn_inputs(wl, layer)
    kc = np.empty((Hkv, R, D), dtype=base["k_ctx"].dtype)
    vc = np.empty_like(kc)
    fill_k = _store(_normal(rng(wl.wid, T_SPARE, layer, 1), (Hkv, R, D)), wl.dtype)
    fill_v = _store(_normal(rng(wl.wid, T_SPARE, layer, 2), (Hkv, R, D)), wl.dtype)
    kc[:], vc[:] = fill_k, fill_v
    src = 0
    for b in range(B):
        n = int(p[b])
        kc[:, start[b]:start[b] + n] = base["k_ctx"][:, src:src + n]
        vc[:, start[b]:start[b] + n] = base["v_ctx"][:, src:src + n]
        src += n
    return dict(q=base["q"], k_blk=base["k_blk"], v_blk=base["v_blk"], k_ctx=kc, v_ctx=vc,
                ctx_start=start, ctx_len=p.astype(np.int32), scale=base["scale"])


def lmhead_inputs(wl: Workload) -> dict:
    """hidden [B*S][H] ~ N(0,1); W [V][H] ~ N(0, w_std^2)."""
    w = wl.wid
    return dict(
        hidden=_store(_normal(rng(w, T_HIDDEN), (wl.M, wl.H)), wl.dtype),
        w=_store(_normal(rng(w, T_W), (wl.V, wl.H), wl.w_std), wl.dtype),
    )


def spikes(wl: Workload) -> dict:
    """One spike per logits row: a token uniform on [0, V) (the mask id included)
    and a height Uniform[0, spike_hi]."""
    w = wl.wid
    tok = rng(w, T_SPIKE_TOK).integers(0, wl.V, size=wl.M).astype(np.int64)
    val = rng(w, T_SPIKE_VAL).uniform(0.0, wl.spike_hi, size=wl.M).astype(np.float32)
    return dict(tok=tok, val=val)


def direct_logits(wl: Workload, noise_std: Optional[float] = None, salt: int = 0) -> np.ndarray:
    """Logits drawn directly (no GEMM): N(0, noise_std^2) noise plus each row's spike,
    float32 [B*S][V]. For workload 0 the noise is N(0,1); for the LM-head workloads the
    default noise_std matches the spread of hidden . W^T, i.e. w_std * sqrt(H)."""
    if noise_std is None:
        noise_std = 1.0 if wl.wid == 0 else wl.w_std * float(np.sqrt(wl.H))
    x = _normal(rng(wl.wid, T_LOGIT_NOISE, 0, salt), (wl.M, wl.V), noise_std)
    sp = spikes(wl)
    x[np.arange(wl.M), sp["tok"]] += sp["val"]
    return x


def initial_state(wl: Workload) -> dict:
    """tokens int32 [B][S] and mask_bits uint64 [B] (bit i set = position i masked).

    Fully masked blocks, except with ``partial_init``: blocks b >= B/2 get k ~ UniformInt[4, 12]
    committed positions (a uniform subset) holding ids uniform on [0, V) without the mask id."""
    B, S = wl.B, wl.S
    tokens = np.full((B, S), wl.mask_id, dtype=np.int32)
    bits = np.zeros(B, dtype=np.uint64)
    full = np.uint64((1 << S) - 1) if S < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
    g = rng(wl.wid, T_MASK_INIT)
    gt = rng(wl.wid, T_MASK_TOK)
    for b in range(B):
        bits[b] = full
        if wl.partial_init and b >= B // 2:
            k = int(g.integers(4, 12, endpoint=True))
            pos = g.choice(S, size=k, replace=False)
            for p in sorted(int(x) for x in pos):
                t = int(gt.integers(0, wl.V - 1))
                if t >= wl.mask_id:
                    t += 1
                tokens[b, p] = t
                bits[b] = np.uint64(int(bits[b]) & ~(1 << p))
    return dict(tokens=tokens, mask_bits=bits)
