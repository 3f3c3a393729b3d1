"""Benchmark of the TwoTower denoiser block step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..4] [--no-cpu-baseline] [--calls-only]

One step = one pass of the whole hot path over one batch of blocks: block attention for every
layer, the LM-head product, the synthetic logit spikes (input construction, not the method),
and confidence unmasking. Steps cycle through the T = 16 steps of a block; at each block
boundary the block state (tokens, mask bits) is reset from a pristine copy. Inputs are seeded
synthetic tensors (synth), uploaded to HBM before the timed region.

The default workload is the largest one that fits one GPU: batch 4, 131072-token prefixes, six
attention layers with separate caches (attention is most of its step).

Prints one JSON line. `value` = denoise block-steps per second over the K timed steps (a
block-step = one step of one block that still had a masked position at the start of the step);
committed tokens/s and per-kernel rooflines ride along. The timed step loop carries no per-call
events; per-call durations are medians over their own loop afterwards (each launch between two
HIP events on the stream the kernels are launched on).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise block-steps/s + committed tokens/s; % HBM roofline (attn), % MFMA (LM head)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
ATTN_KERNELS = "attn_partial + attn_combine"
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4],
                    help="1-4: the batch-1 2K, batch-8 8K, ragged batch-32 and batch-4 128K six-layer workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calls-only", action="store_true",
                    help="skip the step loops and the CPU baseline: per-call medians only (every unmasking "
                         "call at step 0), for kernel traces of single calls; prints a per-call JSON line, "
                         "not the benchmark line")
    ap.add_argument("--cpu-steps", type=int, default=2, help="oracle block-steps in the CPU sample")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run a 1 GiB device copy first (calibrates HBM byte counters)")
    ap.add_argument("--share", action="store_true",
                    help="instead of the step: time the kernels at one GPU's share of an 8-way split "
                         "(LM head over a 16384-row vocabulary shard, attention over one kv head)")
    return ap.parse_args()


def share(torch, bmd):
    """One GPU's share of an 8-way split, timed on this GPU: the LM head over a 16384-row vocabulary
    shard (H = 2688, 16 to 512 hidden rows) and attention over one kv head (16 query heads) at
    batch 4 x 131072-token prefixes. N(0,1) inputs (W scaled by 0.02), median of 30 calls with
    events on the current stream."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(8)

    def median_us(fn, n=30, warm=5):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record()
        for k in range(n):
            fn()
            ev[k + 1].record()
        torch.cuda.synchronize()
        t = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(n))
        return t[n // 2] * 1e3

    rows = []
    H, V = 2688, 131072 // 8
    w = (torch.randn(V, H, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    for M in (16, 64, 128, 512):
        hid = torch.randn(M, H, device=dev, generator=g).to(torch.bfloat16)
        out = torch.empty(M, V, device=dev)
        us = median_us(lambda: bmd.tt_lmhead_logits(hid, w, out))
        byts = 2.0 * V * H + 2.0 * M * H + 4.0 * M * V
        rows.append({"call": "tt_lmhead_logits", "M": M, "H": H, "V": V, "us": round(us, 2),
                     "GB_s": round(byts / us / 1e3, 1), "TFLOP_s": round(2.0 * M * H * V / us / 1e6, 1)})
    del w, hid, out
    B, S, Hq, Hkv, D, P = 4, 16, 16, 1, 128, 131072
    q, kb, vb = (torch.randn(*sh, device=dev, generator=g).to(torch.bfloat16)
                 for sh in ((B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D)))
    kc = torch.randn(Hkv, B * P, D, device=dev, generator=g).to(torch.bfloat16)
    vc = torch.randn(Hkv, B * P, D, device=dev, generator=g).to(torch.bfloat16)
    cs = torch.arange(B, dtype=torch.int32, device=dev) * P
    cl = torch.full((B,), P, dtype=torch.int32, device=dev)
    ws = torch.empty(bmd.workspace_bytes("tt_block_attn", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, ctx_rows=B * P,
                                         max_prefix=P), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    us = median_us(lambda: bmd.tt_block_attn(q, kb, vb, kc, vc, cs, cl, max_prefix=P, out=o, workspace=ws))
    byts = 2.0 * (2 * Hkv * B * P * D + 2 * B * S * Hq * D + 2 * B * S * Hkv * D)
    rows.append({"call": "tt_block_attn", "B": B, "prefix": P, "Hq": Hq, "Hkv": Hkv, "D": D, "us": round(us, 2),
                 "GB_s": round(byts / us / 1e3, 1)})
    return {"metric": "kernels at one GPU's share of an 8-way split", "n_gpus": 1, "data": "synthetic",
            "dtype": "bf16", "share": rows}


def algorithmic(wl):
    """Algorithmic bytes / flops per call at this workload (attention: one layer). Attention bytes:
    the context K/V rows read once, Q, the block's K/V, and the output. LM head: W, hidden and
    the fp32 logits written. Split-K partials are overhead and not counted."""
    e = 2 if wl.dtype == "bf16" else 4
    B, S, Hq, Hkv, D, G = wl.B, wl.S, wl.Hq, wl.Hkv, wl.D, wl.G
    sumP = float(sum(wl.prefixes))
    attn_bytes = e * (2 * Hkv * sumP * D + 2 * B * S * Hq * D + 2 * B * S * Hkv * D)
    attn_flops = 4.0 * S * G * D * Hkv * (sumP + B * S)
    lm_bytes = e * (wl.V * wl.H + wl.M * wl.H) + 4.0 * wl.M * wl.V
    lm_flops = 2.0 * wl.M * wl.H * wl.V
    return dict(attn_bytes=attn_bytes, attn_flops=attn_flops, lm_bytes=lm_bytes, lm_flops=lm_flops)


TRAFFIC_SOURCES = {"lmhead": ("lmhead.hip", "gemm.hip", "lmhead_int.h", "reduce_int.h", "common.h"),
                   "attn": ("attn.hip", "common.h"),
                   "unmask": ("unmask.hip", "lmhead_int.h", "reduce_int.h", "common.h")}


def read_traffic(kind, wid):
    """HBM bytes per call of `kind` ("lmhead" or "attn") from the committed counter summary
    profiles/<kind>_w<wid>_traffic.txt, if it was taken at this workload and on the current
    kernel code; else None."""
    try:
        kv = {}
        for line in open(os.path.join(ROOT, "profiles", f"{kind}_w{wid}_traffic.txt")):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != source_hash(kind) or kv.get("workload") != f"w{wid}":
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def source_hash(kind):
    """sha256 of a kernel's code (its .hip file and the headers it includes) with // comments,
    trailing blanks and blank lines removed, so that editing a comment does not void a traffic
    record."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kind]:
        text = open(os.path.join(ROOT, "block_mask_diffusion_amd", "csrc", f)).read()
        for line in text.splitlines():
            line = re.sub(r"//.*$", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def cpu_baseline(wl, host, steps):
    """The oracle, as it stands, on a bounded sample: `steps` block-steps of sequence 0
    (every layer's attention for its kv heads, its S LM-head rows, its unmask)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas_name = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:  # noqa: BLE001
        blas_name = "unknown"
    S = wl.S
    layers = []
    for inp in host["attn"]:
        a, n = int(inp["ctx_start"][0]), int(inp["ctx_len"][0])
        layers.append(dict(q=inp["q"][:1], k_blk=inp["k_blk"][:1], v_blk=inp["v_blk"][:1],
                           k_ctx=inp["k_ctx"][:, a:a + n], v_ctx=inp["v_ctx"][:, a:a + n],
                           ctx_start=np.array([0], np.int32), ctx_len=np.array([n], np.int32),
                           scale=inp["scale"]))
    tokens, bits = host["tokens"][:1].copy(), host["bits"][:1].copy()
    t0 = time.perf_counter()
    for step in range(steps):
        r = oracle.denoise_step(layers, host["hidden"][:S], host["w"], wl.dtype, host["spike_tok"][:S],
                                host["spike_val"][:S], tokens, bits, S, step % wl.T, wl.T, wl.gamma, wl.mask_id)
        tokens, bits = r["tokens"], r["mask_bits"]
    dt = time.perf_counter() - t0
    return {"value": steps / dt, "unit": "block-steps/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{steps} block-steps of sequence 0 (all {len(layers)} attention layer(s), "
                      f"{S} LM-head rows, unmask) with numpy fp64; host has {os.cpu_count()} CPUs, "
                      f"BLAS {blas_name}, {blas_threads} threads",
            "seconds": dt}


def lmhead_kernel_name(M, H, V, dtype="bf16"):
    """The kernel tt_lmhead_logits launches for these sizes: the library's own choice (lmhead.hip,
    lm_use_lds / lm_bf16; gemm.hip, gemm_cfg) written out, for the roofline's label. The GEMM's
    template arguments are <waves along M, MFMA tiles per wave along M, along the vocabulary>."""
    if dtype != "bf16":
        return "lmhead_kernel"
    if H % 64 == 0 and (M <= 16 or (M <= 128 and (V + 511) // 512 <= 64 and V * M <= 1 << 21)):
        return "lmhead_lds_kernel"
    if M > 16 and H % 64 == 0:
        if (V + 511) // 512 <= 64 or M > 128:
            return "lmhead_gemm_kernel<2, 4, 4>"      # 256 x 256 tile
        return "lmhead_gemm_kernel<1, 2, 2>" if M <= 64 else "lmhead_gemm_kernel<1, 4, 4>"
    return "lmhead_kernel"


def median_us(torch, stream, fn, n, warm=5, before=None):
    """Median duration of fn() over n launches after `warm` untimed ones, each bracketed by its own
    pair of HIP events on `stream` (the stream the library launches on). before(i), if given, runs
    ahead of launch i outside its events (state resets)."""
    for i in range(warm):
        if before:
            before(i)
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        if before:
            before(i)
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path is built and measured "
              "on a single MI355X", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import block_mask_diffusion_amd as bmd

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.share:
        print(json.dumps(share(torch, bmd)))
        return
    wl = synth.workload(args.workload)
    dev = torch.device("cuda")

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
        if x.dtype == np.uint64:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int64)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    want_cpu = not args.no_cpu_baseline
    t_gen = time.perf_counter()
    host = {"attn": []}
    attn_d = []
    for layer in range(wl.layers):
        inp = synth.attn_inputs(wl, layer)
        attn_d.append({k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()})
        if want_cpu:
            host["attn"].append(inp)
        del inp
    lm = synth.lmhead_inputs(wl)
    hidden_d, w_d = up(lm["hidden"]), up(lm["w"])
    sp = synth.spikes(wl)
    st0 = synth.initial_state(wl)
    if want_cpu:
        host.update(hidden=lm["hidden"], w=lm["w"], spike_tok=sp["tok"], spike_val=sp["val"],
                    tokens=st0["tokens"], bits=st0["mask_bits"])
    del lm
    gen_s = time.perf_counter() - t_gen
    print(f"bench: workload w{wl.wid} ({wl.name}) inputs ready in {gen_s:.1f} s", file=sys.stderr, flush=True)

    # synthetic spikes: one entry per logits row, added with a single scatter_add_ on the flat view
    spk_idx_d = torch.from_numpy(np.arange(wl.M, dtype=np.int64) * wl.V + sp["tok"]).to(dev)
    spk_val_d = torch.from_numpy(sp["val"]).to(dev)
    spk_tok_d = torch.from_numpy(sp["tok"].astype(np.int32)).to(dev)
    tok0_d, bits0_d = up(st0["tokens"]), up(st0["mask_bits"])
    tokens_d, bits_d = tok0_d.clone(), bits0_d.clone()
    logits_d = torch.empty((wl.M, wl.V), dtype=torch.float32, device=dev)
    attn_out = [torch.empty_like(a["q"]) for a in attn_d]
    K, Wm = args.steps, args.warmup
    nm_hist = torch.zeros((K, wl.B), dtype=torch.int32, device=dev)
    nm_hist_fu = torch.zeros((K, wl.B), dtype=torch.int32, device=dev)
    nm_scratch = torch.zeros((wl.B,), dtype=torch.int32, device=dev)
    ws_attn = torch.empty(bmd.workspace_bytes("tt_block_attn", B=wl.B, S=wl.S, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                                              ctx_rows=wl.ctx_rows, max_prefix=wl.max_prefix),
                          dtype=torch.uint8, device=dev)
    ws_um = torch.zeros(max(256, bmd.workspace_bytes("tt_confidence_unmask", B=wl.B, S=wl.S, V=wl.V)),
                        dtype=torch.uint8, device=dev)
    ws_fu = torch.zeros(max(256, bmd.workspace_bytes("tt_lmhead_unmask", B=wl.B, S=wl.S, H=wl.H, V=wl.V)),
                        dtype=torch.uint8, device=dev)

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()

    def attn(layer):
        a = attn_d[layer]
        bmd.tt_block_attn(a["q"], a["k_blk"], a["v_blk"], a["k_ctx"], a["v_ctx"], a["ctx_start"], a["ctx_len"],
                          max_prefix=wl.max_prefix, softmax_scale=a["scale"], out=attn_out[layer], workspace=ws_attn)

    def lmhead():
        bmd.tt_lmhead_logits(hidden_d, w_d, logits_d)

    def spikes():
        logits_d.view(-1).scatter_add_(0, spk_idx_d, spk_val_d)  # synthetic spikes (one per row)

    def unmask(s, nm_out):
        bmd.tt_confidence_unmask(logits_d, tokens_d, bits_d, nm_out, s, wl.T, wl.gamma, wl.mask_id,
                                 workspace=ws_um)

    def fused(s, nm_out):
        bmd.tt_lmhead_unmask(hidden_d, w_d, tokens_d, bits_d, nm_out, s, wl.T, wl.gamma, wl.mask_id,
                             bias_tok=spk_tok_d, bias_val=spk_val_d, workspace=ws_fu)

    def reset():
        tokens_d.copy_(tok0_d)
        bits_d.copy_(bits0_d)

    def step(t, nm_out):
        s = t % wl.T
        if s == 0:
            reset()
        for layer in range(wl.layers):
            attn(layer)
        lmhead()
        spikes()
        unmask(s, nm_out)

    # the fused leg: the same step with tt_lmhead_unmask in place of LM head + spikes + unmask
    # (the spikes enter as its one-entry-per-row logit bias; the logits are never stored)
    def step_fused(t, nm_out):
        s = t % wl.T
        if s == 0:
            reset()
        for layer in range(wl.layers):
            attn(layer)
        fused(s, nm_out)

    def timed_loop(fn, hist):
        for t in range(Wm):
            fn(t, nm_scratch)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record(stream)
        for t in range(K):
            fn(t, hist[t])
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end), time.perf_counter() - t_wall

    if not args.calls_only:
        total_ms, wall = timed_loop(step, nm_hist)
        total_ms_fu, _ = timed_loop(step_fused, nm_hist_fu)
        print(f"bench: timed loops done ({total_ms / K:.3f} ms/step three-call, {total_ms_fu / K:.3f} fused)",
              file=sys.stderr, flush=True)

    # per-call medians, each call launched alone between two events: attention cycles through the
    # layers (each layer's cache is cold again by its next turn at the six-layer workload); the
    # unmask calls start from the step-0 state (every masked row read), reset outside the events
    NC = max(20, K)
    t_attn = median_us(torch, stream, lambda i: attn(i % wl.layers), NC)
    t_lm = median_us(torch, stream, lambda i: lmhead(), NC)
    t_spk = median_us(torch, stream, lambda i: spikes(), NC)
    t_um = median_us(torch, stream, lambda i: unmask(0, nm_scratch), NC, before=lambda i: reset())
    t_fu = median_us(torch, stream, lambda i: fused(0, nm_scratch), NC, before=lambda i: reset())

    # the context tower's step over a committed block (once per block in the outer loop, not part
    # of the denoiser step): one layer's tt_context_extend on layer 0's cache, laid out again with
    # room for S more rows per sequence; ctx_len is restored before every call
    a0 = attn_d[0]
    cap = torch.from_numpy(np.asarray(wl.prefixes, dtype=np.int64) + wl.S)
    ext_start = (torch.cumsum(cap, 0) - cap).to(torch.int32).to(dev)
    rows_old = torch.cat([torch.arange(int(s0), int(s0) + p) for s0, p in zip(wl.ctx_start, wl.prefixes)])
    rows_new = torch.cat([torch.arange(int(s0), int(s0) + p) for s0, p in zip(ext_start.cpu(), wl.prefixes)])
    R2 = int(cap.sum())
    kc2 = torch.zeros((wl.Hkv, R2, wl.D), dtype=a0["k_ctx"].dtype, device=dev)
    vc2 = torch.zeros_like(kc2)
    kc2[:, rows_new.to(dev)] = a0["k_ctx"][:, rows_old.to(dev)]
    vc2[:, rows_new.to(dev)] = a0["v_ctx"][:, rows_old.to(dev)]
    len0 = a0["ctx_len"].clone()
    ext_len = len0.clone()
    ext_out = torch.empty_like(a0["q"])
    ws_ext = torch.empty(bmd.workspace_bytes("tt_block_attn", B=wl.B, S=wl.S, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                                             ctx_rows=R2, max_prefix=wl.max_prefix), dtype=torch.uint8, device=dev)

    def ext(i):
        bmd.tt_context_extend(a0["q"], a0["k_blk"], a0["v_blk"], kc2, vc2, ext_start, ext_len,
                              max_prefix=wl.max_prefix, softmax_scale=a0["scale"], out=ext_out, workspace=ws_ext)

    t_ext = median_us(torch, stream, ext, NC, before=lambda i: ext_len.copy_(len0))
    del kc2, vc2

    # block-steps and commits from the per-step n_masked record
    init_masked = np.array([bin(int(b)).count("1") for b in st0["mask_bits"]])

    def tally(nm):
        block_steps, commits = 0, 0
        for t in range(K):
            start_masked = init_masked if t % wl.T == 0 else nm[t - 1]
            block_steps += int(np.sum(start_masked > 0))
            commits += int(np.sum(start_masked - nm[t]))
        return block_steps, commits

    alg = algorithmic(wl)
    lm_gbs = alg["lm_bytes"] / (t_lm * 1e-6) / 1e9
    lm_tfs = alg["lm_flops"] / (t_lm * 1e-6) / 1e12
    # context extend: the attention's bytes plus the appended rows written
    ext_bytes = alg["attn_bytes"] + (2 if wl.dtype == "bf16" else 4) * 2.0 * wl.B * wl.S * wl.Hkv * wl.D
    attn_gbs = alg["attn_bytes"] / (t_attn * 1e-6) / 1e9
    attn_tfs = alg["attn_flops"] / (t_attn * 1e-6) / 1e12
    um_bytes = 4.0 * wl.V * int(init_masked.sum())
    um_gbs = um_bytes / (t_um * 1e-6) / 1e9
    # attainable LM-head rate: min(MFMA peak, arithmetic intensity x HBM peak)
    lm_attain_tfs = min(MFMA_BF16_PEAK_TFS, alg["lm_flops"] / alg["lm_bytes"] * HBM_PEAK_GBS / 1e3)

    per_step = {"attn": t_attn * wl.layers, "lmhead": t_lm, "unmask": t_um}
    dominant = max(per_step, key=per_step.get)
    if dominant == "lmhead":
        traffic = read_traffic("lmhead", wl.wid)
        lm_kernel = lmhead_kernel_name(wl.M, wl.H, wl.V, wl.dtype)
        ridge = MFMA_BF16_PEAK_TFS * 1e3 / HBM_PEAK_GBS  # flop per byte where the two roofs meet
        if alg["lm_flops"] / alg["lm_bytes"] >= ridge:
            roof = {"kernel": f"{lm_kernel} (tt_lmhead_logits)", "bound": "mfma", "achieved": round(lm_tfs, 1),
                    "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(lm_tfs / MFMA_BF16_PEAK_TFS, 4),
                    "traffic": traffic, "algorithmic_flops": alg["lm_flops"], "avg_launch_us": round(t_lm, 2)}
        else:
            roof = {"kernel": f"{lm_kernel} (tt_lmhead_logits)", "bound": "hbm", "achieved": round(lm_gbs, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "algorithmic_bytes": alg["lm_bytes"], "avg_launch_us": round(t_lm, 2)}
    elif dominant == "attn":
        roof = {"kernel": f"{ATTN_KERNELS} (tt_block_attn, one layer)", "bound": "hbm",
                "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": read_traffic("attn", wl.wid),
                "algorithmic_bytes": alg["attn_bytes"], "avg_launch_us": round(t_attn, 2)}
    else:
        roof = {"kernel": "unmask (tt_confidence_unmask)", "bound": "hbm", "achieved": round(um_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(um_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes": um_bytes, "avg_launch_us": round(t_um, 2)}

    kernels = {
        "attn": {"us_per_layer": round(t_attn, 2), "GB_s": round(attn_gbs, 1),
                 "hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4), "TFLOP_s": round(attn_tfs, 1),
                 "mfma_frac": round(attn_tfs / MFMA_BF16_PEAK_TFS, 4)},
        "lmhead": {"kernel": lmhead_kernel_name(wl.M, wl.H, wl.V, wl.dtype), "us": round(t_lm, 2),
                   "GB_s": round(lm_gbs, 1), "hbm_frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                   "TFLOP_s": round(lm_tfs, 2), "mfma_frac": round(lm_tfs / MFMA_BF16_PEAK_TFS, 4),
                   "attainable_frac": round(lm_tfs / lm_attain_tfs, 4)},
        "unmask": {"us_step0": round(t_um, 2), "masked_rows_step0": int(init_masked.sum()),
                   "GB_s": round(um_gbs, 1), "hbm_frac": round(um_gbs / HBM_PEAK_GBS, 4)},
        "spikes_us": round(t_spk, 2),
        "lmhead_unmask_us_step0": round(t_fu, 2),
        "context_extend_us": round(t_ext, 2),
    }
    per_call = f"median of {NC} launches after 5 warm-ups, each between two HIP events on the launch stream"
    if args.calls_only:
        print(json.dumps({"per_call_only": True, "config": {"workload": f"w{wl.wid}: {wl.name}"},
                          "kernels": kernels, "timing": {"per_call": per_call}}), flush=True)
        return

    block_steps, commits = tally(nm_hist.cpu().numpy())
    block_steps_fu, commits_fu = tally(nm_hist_fu.cpu().numpy())
    sec, sec_fu = total_ms / 1e3, total_ms_fu / 1e3

    cpu = None
    if want_cpu:
        print("bench: CPU baseline (the oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, host, args.cpu_steps)
        cpu.pop("seconds", None)

    out = {
        "metric": METRIC,
        "value": round(block_steps / sec, 2),
        "unit": "block-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded normal Q/K/V, hidden, W~N(0,0.02^2), uniform logit spikes)",
        "config": {"workload": f"w{wl.wid}: {wl.name}", "batch": wl.B, "block": wl.S, "prefix_max": wl.max_prefix,
                   "prefix_sum": wl.ctx_rows, "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.D,
                   "hidden": wl.H, "vocab": wl.V, "layers": wl.layers, "steps_per_block": wl.T,
                   "gamma": wl.gamma, "mask_id": wl.mask_id},
        "committed_tokens_per_s": round(commits / sec, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": {k: v for k, v in kernels.items() if k not in ("lmhead_unmask_us_step0", "context_extend_us")},
        "fused_path": {
            "what": "same step with tt_lmhead_unmask (LM head with the vocabulary reduction in its epilogue, "
                    "spikes as its logit bias, logits never stored) in place of LM head + spikes + unmask",
            "block_steps_per_s": round(block_steps_fu / sec_fu, 2),
            "committed_tokens_per_s": round(commits_fu / sec_fu, 2),
            "ms_per_step": round(total_ms_fu / K, 4),
            "lmhead_unmask_us_step0": round(t_fu, 2),
            "lmhead_unmask_hbm_frac": round((alg["lm_bytes"] - 4.0 * wl.M * wl.V) / (t_fu * 1e-6) / 1e9
                                            / HBM_PEAK_GBS, 4),
            "lmhead_unmask_mfma_frac": round(alg["lm_flops"] / (t_fu * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        },
        "context_extend": {
            "what": "tt_context_extend, one layer: causal attention of the S committed tokens over "
                    "[cache ; block], then the append of their K/V (once per block, not in the step)",
            "us": round(t_ext, 2),
            "GB_s": round(ext_bytes / (t_ext * 1e-6) / 1e9, 1),
            "hbm_frac": round(ext_bytes / (t_ext * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "timing": {"per_call": per_call + ", after the step loops",
                   "step_loop": f"{K} steps between two events, no per-call events inside"},
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
