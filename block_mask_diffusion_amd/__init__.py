"""TwoTower denoiser block step on AMD CDNA4 (gfx950).

Python face of libtt.so: the calls of include/tt.h under the same names, taking torch tensors.
This layer only marshals arguments (shapes, dtypes, pointers, the current HIP stream, workspace
allocation); every step of the computation runs in the HIP kernels of the library.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib
from ._lib import TTError, TT_BF16, TT_F32

__all__ = ["tt_block_attn", "tt_context_extend", "tt_lmhead_logits", "tt_confidence_unmask",
           "tt_confidence_unmask_noalloc", "tt_unmask_sample", "tt_lmhead_unmask", "workspace_bytes", "TTError",
           "abi_version"]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TT_BF16
    if t.dtype == torch.float32:
        return TT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check(status: int, what: str):
    if status != _lib.TT_OK:
        raise TTError(status, what)


def _dev(*ts):
    for t in ts:
        if t is not None:
            _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous and on the GPU")


def abi_version() -> int:
    return _lib.load().tt_abi_version()


def workspace_bytes(fn: str, **kw) -> int:
    """Workspace size of `tt_block_attn` / `tt_confidence_unmask` / `tt_lmhead_unmask` for the
    given sizes (a pure host computation: nothing is launched)."""
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    if fn == "tt_block_attn":
        one = ctypes.c_void_p(16)  # non-null placeholders: a size query dereferences nothing
        st = lib.tt_block_attn(one, one, one, one, one, one, one, one, kw["B"], kw["S"], kw["Hq"],
                               kw["Hkv"], kw["D"], kw.get("ctx_rows", 0), kw["max_prefix"],
                               kw.get("softmax_scale", 1.0 / math.sqrt(kw["D"])),
                               kw.get("dtype", TT_BF16), None, ctypes.byref(n), None)
    elif fn == "tt_confidence_unmask":
        one = ctypes.c_void_p(16)
        st = lib.tt_confidence_unmask(one, one, one, one, None, None, kw["B"], kw["S"], kw["V"], 0, 1,
                                      0.5, kw.get("mask_id", 0), None, ctypes.byref(n), None)
    elif fn == "tt_lmhead_unmask":
        one = ctypes.c_void_p(16)
        st = lib.tt_lmhead_unmask(one, one, None, None, one, one, one, None, None, kw["B"], kw["S"], kw["H"],
                                  kw["V"], 0, 1, ctypes.byref(_sampler("confidence", 0.5, 1.0)),
                                  kw.get("mask_id", 0), kw.get("dtype", TT_BF16), None, ctypes.byref(n), None)
    else:
        raise ValueError(fn)
    _check(st, fn)
    return n.value


def _sampler(kind: str, gamma: float, temperature: float) -> "_lib.Sampler":
    _need(kind in _lib.SAMPLER_KINDS, f"sampler kind is one of {sorted(_lib.SAMPLER_KINDS)}")
    return _lib.Sampler(_lib.SAMPLER_KINDS[kind], float(gamma), float(temperature))


def _workspace(nbytes: int, workspace: Optional[torch.Tensor], device, zeroed: bool = False) -> torch.Tensor:
    """A caller's workspace, checked for size, or a new one (zero-filled when `zeroed`: the
    unmasking calls keep arrival counters, zero between calls, at its start)."""
    if workspace is not None:
        _need(workspace.is_cuda and workspace.numel() * workspace.element_size() >= nbytes,
              "workspace too small")
        return workspace
    alloc = torch.zeros if zeroed else torch.empty
    return alloc(max(nbytes, 256), dtype=torch.uint8, device=device)


def tt_block_attn(q: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor,
                  k_ctx: torch.Tensor, v_ctx: torch.Tensor, ctx_start: torch.Tensor,
                  ctx_len: torch.Tensor, max_prefix: int, softmax_scale: Optional[float] = None,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Block attention of one layer (see include/tt.h). q [B][S][Hq][D], k_blk/v_blk
    [B][S][Hkv][D], k_ctx/v_ctx [Hkv][ctx_rows][D], ctx_start/ctx_len int32 [B]."""
    _need(q.dim() == 4 and k_blk.dim() == 4 and v_blk.dim() == 4, "q, k_blk, v_blk are 4-d")
    B, S, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    _need(tuple(k_blk.shape) == (B, S, Hkv, D) and tuple(v_blk.shape) == (B, S, Hkv, D), "block K/V shape")
    _need(k_ctx.dim() == 3 and tuple(k_ctx.shape) == tuple(v_ctx.shape), "context K/V shape")
    _need(k_ctx.shape[0] == Hkv and k_ctx.shape[2] == D, "context K/V shape")
    _need(ctx_start.dtype == torch.int32 and ctx_len.dtype == torch.int32, "ctx_start/ctx_len are int32")
    _need(ctx_start.numel() == B and ctx_len.numel() == B, "ctx_start/ctx_len have B entries")
    for t in (k_blk, v_blk, k_ctx, v_ctx):
        _need(t.dtype == q.dtype, "all attention tensors share one dtype")
    _dev(q, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, out)
    if out is None:
        out = torch.empty_like(q)
    _dev(out)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    dt = _dtype(q)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    args = [_ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_start), _ptr(ctx_len),
            _ptr(out), B, S, Hq, Hkv, D, k_ctx.shape[1], int(max_prefix), scale, dt]
    _check(lib.tt_block_attn(*args, None, ctypes.byref(n), None), "tt_block_attn")
    ws = _workspace(n.value, workspace, q.device)
    n2 = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check(lib.tt_block_attn(*args, _ptr(ws), ctypes.byref(n2), _stream(stream)), "tt_block_attn")
    return out


def tt_context_extend(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      k_ctx: torch.Tensor, v_ctx: torch.Tensor, ctx_start: torch.Tensor,
                      ctx_len: torch.Tensor, max_prefix: int, softmax_scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """The context tower's causal attention over a committed block, then the append of k_new /
    v_new to the cache (k_ctx, v_ctx and ctx_len updated in place; see include/tt.h). Shapes as
    tt_block_attn with k_new / v_new [B][S][Hkv][D]."""
    _need(q.dim() == 4 and k_new.dim() == 4 and v_new.dim() == 4, "q, k_new, v_new are 4-d")
    B, S, Hq, D = q.shape
    Hkv = k_new.shape[2]
    _need(tuple(k_new.shape) == (B, S, Hkv, D) and tuple(v_new.shape) == (B, S, Hkv, D), "new K/V shape")
    _need(k_ctx.dim() == 3 and tuple(k_ctx.shape) == tuple(v_ctx.shape), "context K/V shape")
    _need(k_ctx.shape[0] == Hkv and k_ctx.shape[2] == D, "context K/V shape")
    _need(ctx_start.dtype == torch.int32 and ctx_len.dtype == torch.int32, "ctx_start/ctx_len are int32")
    _need(ctx_start.numel() == B and ctx_len.numel() == B, "ctx_start/ctx_len have B entries")
    for t in (k_new, v_new, k_ctx, v_ctx):
        _need(t.dtype == q.dtype, "all attention tensors share one dtype")
    _dev(q, k_new, v_new, k_ctx, v_ctx, ctx_start, ctx_len, out)
    if out is None:
        out = torch.empty_like(q)
    _dev(out)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    args = [_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_start), _ptr(ctx_len),
            _ptr(out), B, S, Hq, Hkv, D, k_ctx.shape[1], int(max_prefix), scale, _dtype(q)]
    _check(lib.tt_context_extend(*args, None, ctypes.byref(n), None), "tt_context_extend")
    ws = _workspace(n.value, workspace, q.device)
    n2 = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check(lib.tt_context_extend(*args, _ptr(ws), ctypes.byref(n2), _stream(stream)), "tt_context_extend")
    return out


def tt_lmhead_logits(hidden: torch.Tensor, w: torch.Tensor, logits: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """logits [M][V] fp32 = hidden [M][H] . w[V][H]^T (see include/tt.h)."""
    _need(hidden.dim() == 2 and w.dim() == 2 and hidden.shape[1] == w.shape[1], "hidden [M][H], w [V][H]")
    _need(hidden.dtype == w.dtype, "hidden and w share one dtype")
    M, H = hidden.shape
    V = w.shape[0]
    if logits is None:
        logits = torch.empty((M, V), dtype=torch.float32, device=hidden.device)
    _need(logits.dtype == torch.float32 and tuple(logits.shape) == (M, V), "logits fp32 [M][V]")
    _dev(hidden, w, logits)
    _check(_lib.load().tt_lmhead_logits(_ptr(hidden), _ptr(w), _ptr(logits), M, H, V, _dtype(hidden),
                                        _stream(stream)), "tt_lmhead_logits")
    return logits


def tt_confidence_unmask(logits: torch.Tensor, tokens: torch.Tensor, mask_bits: torch.Tensor,
                         n_masked: torch.Tensor, step: int, num_steps: int, gamma: float,
                         mask_id: int, conf_out: Optional[torch.Tensor] = None,
                         pred_out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """One confidence-unmasking step, in place on tokens int32 [B][S] and mask_bits (64-bit) [B];
    writes n_masked int32 [B] (see include/tt.h)."""
    _need(tokens.dim() == 2 and tokens.dtype == torch.int32, "tokens int32 [B][S]")
    B, S = tokens.shape
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.shape[0] == B * S, "logits fp32 [B*S][V]")
    V = logits.shape[1]
    _unmask_io(B, S, tokens, mask_bits, n_masked, conf_out, pred_out)
    _dev(logits, tokens, mask_bits, n_masked, conf_out, pred_out)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    args = [_ptr(logits), _ptr(tokens), _ptr(mask_bits), _ptr(n_masked), _ptr(conf_out), _ptr(pred_out),
            B, S, V, int(step), int(num_steps), float(gamma), int(mask_id)]
    _check(lib.tt_confidence_unmask(*args, None, ctypes.byref(n), None), "tt_confidence_unmask")
    ws = _workspace(n.value, workspace, logits.device, zeroed=True)
    n2 = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check(lib.tt_confidence_unmask(*args, _ptr(ws), ctypes.byref(n2), _stream(stream)), "tt_confidence_unmask")


def tt_confidence_unmask_noalloc(logits: torch.Tensor, tokens: torch.Tensor, mask_bits: torch.Tensor,
                                 n_masked: torch.Tensor, step: int, num_steps: int, gamma: float,
                                 mask_id: int, conf_out: Optional[torch.Tensor] = None,
                                 pred_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """tt_confidence_unmask without a workspace: the library's per-device scratch serves instead,
    and nothing is allocated (see include/tt.h for its size limit and its sharing rule)."""
    _need(tokens.dim() == 2 and tokens.dtype == torch.int32, "tokens int32 [B][S]")
    B, S = tokens.shape
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.shape[0] == B * S, "logits fp32 [B*S][V]")
    V = logits.shape[1]
    _unmask_io(B, S, tokens, mask_bits, n_masked, conf_out, pred_out)
    _dev(logits, tokens, mask_bits, n_masked, conf_out, pred_out)
    _check(_lib.load().tt_confidence_unmask_noalloc(
        _ptr(logits), _ptr(tokens), _ptr(mask_bits), _ptr(n_masked), _ptr(conf_out), _ptr(pred_out), B, S, V,
        int(step), int(num_steps), float(gamma), int(mask_id), _stream(stream)), "tt_confidence_unmask_noalloc")


def tt_unmask_sample(logits: torch.Tensor, tokens: torch.Tensor, mask_bits: torch.Tensor,
                     n_masked: torch.Tensor, step: int, num_steps: int, mask_id: int,
                     sampler: str = "confidence", gamma: float = 0.8, temperature: float = 1.0,
                     conf_out: Optional[torch.Tensor] = None, pred_out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """One unmasking step with a chosen sampler ("confidence" or "predict_noise") and softmax
    temperature, in place on tokens / mask_bits (see include/tt.h)."""
    _need(tokens.dim() == 2 and tokens.dtype == torch.int32, "tokens int32 [B][S]")
    B, S = tokens.shape
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.shape[0] == B * S, "logits fp32 [B*S][V]")
    V = logits.shape[1]
    _unmask_io(B, S, tokens, mask_bits, n_masked, conf_out, pred_out)
    _dev(logits, tokens, mask_bits, n_masked, conf_out, pred_out)
    sm = _sampler(sampler, gamma, temperature)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    args = [_ptr(logits), _ptr(tokens), _ptr(mask_bits), _ptr(n_masked), _ptr(conf_out), _ptr(pred_out),
            B, S, V, int(step), int(num_steps), ctypes.byref(sm), int(mask_id)]
    _check(lib.tt_unmask_sample(*args, None, ctypes.byref(n), None), "tt_unmask_sample")
    ws = _workspace(n.value, workspace, logits.device, zeroed=True)
    n2 = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check(lib.tt_unmask_sample(*args, _ptr(ws), ctypes.byref(n2), _stream(stream)), "tt_unmask_sample")


def _unmask_io(B: int, S: int, tokens, mask_bits, n_masked, conf_out, pred_out):
    _need(mask_bits.dtype in (torch.int64, torch.uint64) and mask_bits.numel() == B, "mask_bits 64-bit [B]")
    _need(n_masked.dtype == torch.int32 and n_masked.numel() == B, "n_masked int32 [B]")
    if conf_out is not None:
        _need(conf_out.dtype == torch.float32 and conf_out.numel() == B * S, "conf_out fp32 [B*S]")
    if pred_out is not None:
        _need(pred_out.dtype == torch.int32 and pred_out.numel() == B * S, "pred_out int32 [B*S]")


def tt_lmhead_unmask(hidden: torch.Tensor, w: torch.Tensor, tokens: torch.Tensor, mask_bits: torch.Tensor,
                     n_masked: torch.Tensor, step: int, num_steps: int, gamma: float, mask_id: int,
                     bias_tok: Optional[torch.Tensor] = None, bias_val: Optional[torch.Tensor] = None,
                     conf_out: Optional[torch.Tensor] = None, pred_out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None, sampler: str = "confidence",
                     temperature: float = 1.0) -> None:
    """LM head + one confidence-unmasking step without materialising the logits (see
    include/tt.h). hidden bf16 [B*S][H], w bf16 [V][H]; tokens int32 [B][S] and mask_bits
    (64-bit) [B] are updated in place; optional one-entry-per-row logit bias bias_tok int32 /
    bias_val fp32 [B*S]; sampler "confidence" (threshold gamma) or "predict_noise", softmax
    temperature."""
    _need(tokens.dim() == 2 and tokens.dtype == torch.int32, "tokens int32 [B][S]")
    B, S = tokens.shape
    _need(hidden.dim() == 2 and w.dim() == 2 and hidden.shape[1] == w.shape[1], "hidden [M][H], w [V][H]")
    _need(hidden.shape[0] == B * S, "hidden has B*S rows")
    _need(hidden.dtype == w.dtype, "hidden and w share one dtype")
    _need((bias_tok is None) == (bias_val is None), "bias_tok and bias_val go together")
    if bias_tok is not None:
        _need(bias_tok.dtype == torch.int32 and bias_tok.numel() == B * S, "bias_tok int32 [B*S]")
        _need(bias_val.dtype == torch.float32 and bias_val.numel() == B * S, "bias_val fp32 [B*S]")
    _unmask_io(B, S, tokens, mask_bits, n_masked, conf_out, pred_out)
    _dev(hidden, w, tokens, mask_bits, n_masked, bias_tok, bias_val, conf_out, pred_out)
    H, V = hidden.shape[1], w.shape[0]
    sm = _sampler(sampler, gamma, temperature)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    args = [_ptr(hidden), _ptr(w), _ptr(bias_tok), _ptr(bias_val), _ptr(tokens), _ptr(mask_bits), _ptr(n_masked),
            _ptr(conf_out), _ptr(pred_out), B, S, H, V, int(step), int(num_steps), ctypes.byref(sm), int(mask_id),
            _dtype(hidden)]
    _check(lib.tt_lmhead_unmask(*args, None, ctypes.byref(n), None), "tt_lmhead_unmask")
    ws = _workspace(n.value, workspace, hidden.device, zeroed=True)
    n2 = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check(lib.tt_lmhead_unmask(*args, _ptr(ws), ctypes.byref(n2), _stream(stream)), "tt_lmhead_unmask")
