#!/usr/bin/env python3
"""Throughput of QK-norm + RoPE + causal GQA attention on one MI355X.

A step is one pass of the whole attention hot path over one batch: the
default workload is the mixed packed step on Qwen3-8B-shaped heads (Hq=32,
Hkv=8, D=128): a prefill of 4 requests x 4096 tokens (QK-norm + RoPE +
K/V-cache write + causal attention) followed, on the same stream, by one
decode step for 128 requests whose caches hold U[1, 16384] entries.

Metric: attention work as a fraction of the MI355X roofline.  For a step,
    value = 100 * (F / P_mfma + B / P_hbm) / t_step
with F the causal prefill FLOPs (sum over requests of 2*D*Hq*T(T+1)), B the
decode K/V bytes (sum over requests of 2*Hkv*(L+1)*D*2), P_mfma = 2500 TFLOP/s
(dense bf16 MFMA) and P_hbm = 8000 GB/s; i.e. the ideal time of the step's
work on each roofline divided by the measured step time.  Inputs are resident
in HBM before timing starts.

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: this path runs on
one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Source of each timed kernel on the bf16 path (with the headers every kernel
# includes): a counter summary applies only to the source it was taken on.
_COMMON = ["decoder_attention_amd/csrc/device_common.h", "decoder_attention_amd/csrc/launch.h"]
KERNEL_SOURCES = {
    "prefill_attn_mfma_bf16": ["decoder_attention_amd/csrc/prefill_mfma.hip", "decoder_attention_amd/csrc/decode_body.h"]
    + _COMMON,
    "prefill_attn_mfma_bf16_shifted": ["decoder_attention_amd/csrc/prefill_mfma.hip",
                                       "decoder_attention_amd/csrc/decode_body.h"] + _COMMON,
    "fused_step_attn": ["decoder_attention_amd/csrc/prefill_mfma.hip", "decoder_attention_amd/csrc/decode_body.h"]
    + _COMMON,
    "decode_attn_split": ["decoder_attention_amd/csrc/decode_mfma.hip", "decoder_attention_amd/csrc/decode_body.h"]
    + _COMMON,
    "decode_attn_combine": ["decoder_attention_amd/csrc/decode_mfma.hip"] + _COMMON,
    "qknorm_rope_kv_prefill": ["decoder_attention_amd/csrc/qknorm_rope.hip"] + _COMMON,
    "qknorm_rope_kv_decode": ["decoder_attention_amd/csrc/qknorm_rope.hip", "decoder_attention_amd/csrc/decode_plan.h"]
    + _COMMON,
    "fused_add_rmsnorm": ["decoder_attention_amd/csrc/layer_ops.hip"] + _COMMON,
    "gather_last": ["decoder_attention_amd/csrc/layer_ops.hip"] + _COMMON,
    "argmax_partial": ["decoder_attention_amd/csrc/layer_ops.hip"] + _COMMON,
}


# The bf16 prefill's two attention kernels: p = 2^s unshifted (plain prefill whose norm weights bound the
# scores) and the running-max one (appends, larger weights).  Both are launched for a plain prefill; the one
# the weights do not select returns at once in every workgroup.
PREFILL_KERNELS = ("prefill_attn_mfma_bf16", "prefill_attn_mfma_bf16_shifted")


def working_prefill_kernel(kernels):
    """The prefill attention kernel that did the work (the larger total time)."""
    names = [k for k in PREFILL_KERNELS if k in kernels]
    return max(names, key=lambda k: kernels[k][0]) if names else None


def prefill_roofline(kernels, F, B, workload):
    name = working_prefill_kernel(kernels)
    rf = roofline_for(name, kernels, F, B, workload)
    others = {k: kernels[k][0] / kernels[k][1] for k in PREFILL_KERNELS if k in kernels and k != name}
    if others:
        rf["other_path_avg_launch_ms"] = others
    return rf


def prefill_flops(seqlens, hq, d) -> float:
    return float(sum(2 * d * hq * t * (t + 1) for t in seqlens))


def append_flops(past_lens, chunk_lens, hq, d) -> float:
    """Chunk token j of request r sees P_r + j + 1 keys: 4*D*Hq FLOP per visible pair."""
    return float(sum(2 * d * hq * (2 * t * p + t * (t + 1)) for p, t in zip(past_lens, chunk_lens)))


def decode_kv_bytes(cache_lens, hkv, d, elem) -> float:
    return float(sum(2 * hkv * (int(L) + 1) * d * elem for L in cache_lens))


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it is for this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    entry = table.get(kernel, {}).get(workload)
    src = KERNEL_SOURCES.get(kernel)
    if not entry or not src or entry.get("source_sha256") != source_digest(src):
        return None
    return entry.get("hbm_bytes_per_launch")


class Runner:
    """Holds device inputs/outputs/workspaces of a workload and issues its step."""

    def __init__(self, w, torch, da, fused: bool = False):
        self.torch, self.da, self.w = torch, da, w
        self.calls = []
        if w.prefill is not None:
            p = w.prefill
            h = p.heads
            cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, p.qkv.dtype, h.rms_eps, h.rope_base)
            out = torch.empty((p.num_tokens, h.num_q_heads * h.head_dim), dtype=p.qkv.dtype, device=p.qkv.device)
            ws_bytes = da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_PREFILL, p.num_tokens, p.max_seqlen)
            ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=p.qkv.device)
            args = (cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens, p.num_tokens,
                    p.num_seqs, p.max_seqlen, p.k_cache, p.v_cache, p.cache_capacity, out, ws, ws_bytes)
            self.calls.append((da.qknorm_rope_attn_prefill, args, (out, ws)))
        if w.append is not None:
            a = w.append
            h = a.heads
            cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, a.qkv.dtype, h.rms_eps, h.rope_base)
            out = torch.empty((a.num_tokens, h.num_q_heads * h.head_dim), dtype=a.qkv.dtype, device=a.qkv.device)
            ws_bytes = da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_PREFILL, a.num_tokens, a.max_seqlen)
            ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=a.qkv.device)
            args = (cfg, a.qkv, a.q_norm_weight, a.k_norm_weight, a.positions, a.cu_seqlens, a.cache_lens,
                    a.num_tokens, a.num_seqs, a.max_seqlen, a.max_cache_len, a.k_cache, a.v_cache,
                    a.cache_capacity, out, ws, ws_bytes)
            self.calls.append((da.qknorm_rope_attn_prefill_append, args, (out, ws)))
        if w.decode is not None:
            d = w.decode
            h = d.heads
            cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, d.qkv.dtype, h.rms_eps, h.rope_base)
            out = torch.empty((d.num_seqs, h.num_q_heads * h.head_dim), dtype=d.qkv.dtype, device=d.qkv.device)
            ws_bytes = da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_DECODE, d.num_seqs, d.max_cache_len)
            ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=d.qkv.device)
            args = (cfg, d.qkv, d.q_norm_weight, d.k_norm_weight, d.positions, d.cache_lens, d.num_seqs,
                    d.max_cache_len, d.k_cache, d.v_cache, d.cache_capacity, out, ws, ws_bytes)
            self.calls.append((da.qknorm_rope_attn_decode, args, (out, ws)))
        if w.norm is not None:
            n = w.norm
            out = torch.empty_like(n.x)
            res = n.residual if n.has_residual else torch.empty_like(n.x)
            args = (da_dtype(da, n.x), n.rms_eps, n.x, res, n.has_residual, n.weight, out, n.x.shape[0],
                    n.x.shape[1])
            self.calls.append((da.qknorm_rope_attn_fused_add_rmsnorm, args, (out, res)))
        if w.next_token is not None:
            nt = w.next_token
            b, c, v = len(nt.seqlens), nt.hidden.shape[1], nt.logits.shape[1]
            last = torch.empty((b, c), dtype=nt.hidden.dtype, device=nt.hidden.device)
            args = (da_dtype(da, nt.hidden), nt.hidden, nt.cu_seqlens, nt.hidden.shape[0], b, c, last)
            self.calls.append((da.qknorm_rope_attn_gather_last, args, (last,)))
            idx = torch.empty((b,), dtype=torch.int32, device=nt.logits.device)
            ws_bytes = da.qknorm_rope_attn_argmax_workspace_bytes(b, v)
            ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=nt.logits.device)
            args = (da_dtype(da, nt.logits), nt.logits, b, v, nt.logits.stride(0), idx, ws, ws_bytes)
            self.calls.append((da.qknorm_rope_attn_argmax, args, (idx, ws)))

        if fused and w.prefill is not None and w.decode is not None:
            # The same step through qknorm_rope_attn_mixed_step: one call, the prefill attention and the decode
            # split in one launch (both halves share the norm weights, as one layer's do).
            (_, pa, pkeep), (_, dargs, dkeep) = self.calls[0], self.calls[1]
            mixed = (pa[0], pa[2], pa[3]) + pa[1:2] + pa[4:] + dargs[1:2] + dargs[4:]
            self.calls = [(da.qknorm_rope_attn_mixed_step, mixed, pkeep + dkeep)] + self.calls[2:]

    def step(self):
        for fn, args, _ in self.calls:
            status = fn(*args)
            if status != 0:
                raise self.da.QkraError(status, fn.__name__)

    def hbm_bytes(self):
        """Algorithmic HBM bytes per launch of the kernels outside the attention roofline."""
        out = {}
        if self.w.norm is not None:
            n = self.w.norm
            row = n.x.shape[1] * n.x.element_size()
            out["fused_add_rmsnorm"] = float(n.x.shape[0] * row * (4 if n.has_residual else 3) + row)
        if self.w.next_token is not None:
            nt = self.w.next_token
            row = nt.hidden.shape[1] * nt.hidden.element_size()
            out["gather_last"] = float(2 * row * sum(1 for t in nt.seqlens if t > 0))
            out["argmax_partial"] = float(nt.logits.shape[0] * nt.logits.shape[1] * nt.logits.element_size())
        return out

    def work(self):
        F = B = 0.0
        if self.w.prefill is not None:
            h = self.w.prefill.heads
            F = prefill_flops(self.w.prefill.seqlens, h.num_q_heads, h.head_dim)
        if self.w.append is not None:
            h = self.w.append.heads
            F += append_flops(self.w.append.past_lens, self.w.append.seqlens, h.num_q_heads, h.head_dim)
        if self.w.decode is not None:
            h = self.w.decode.heads
            B = decode_kv_bytes(self.w.decode.cache_lens.tolist(), h.num_kv_heads, h.head_dim,
                                self.w.decode.qkv.element_size())
        return F, B


def da_dtype(da, t):
    return da.QKRA_BF16 if str(t.dtype) == "torch.bfloat16" else da.QKRA_FP32


def _timed_region(runner, steps: int) -> float:
    torch = runner.torch
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        runner.step()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def single_step_ms(runner, reps: int, evict: bool) -> float:
    """Mean time of one step run alone (synchronised before and after, its own
    events).  With `evict`, each step follows a 1 GiB read, outside the
    events, that leaves none of the step's data in the 256 MB last-level
    cache; without it the same protocol measures the warm step, so that the
    two differ by the cache alone."""
    torch = runner.torch
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    total = 0.0
    for _ in range(reps):
        if evict:
            scratch.sum()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        runner.step()
        stop.record()
        torch.cuda.synchronize()
        total += start.elapsed_time(stop)
    del scratch
    return total / reps


def cache_effect(runner, reps: int = 10) -> dict:
    warm = single_step_ms(runner, reps, False)
    cold = single_step_ms(runner, reps, True)
    return {"ms_single_step_warm": warm, "ms_single_step_after_1gib_read": cold}


def time_steps(runner, steps: int, warmup: int):
    """Warm-up steps, then two timed regions of `steps` steps each.

    In the first region the library brackets every kernel launch with a pair
    of HIP events on the launch stream (which adds a little time between
    launches); it gives each kernel's average launch duration.  The second
    region is the step as a caller runs it: its time per step is the
    benchmark's (it comes second so that the GPU is fully warm by then).
    Returns (ms per step, ms per step with per-kernel events, kernel table).
    """
    torch, da = runner.torch, runner.da
    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    da.qknorm_rope_attn_read_kernel_timing()          # drop anything recorded before
    da.qknorm_rope_attn_set_kernel_timing(True)
    ms_events = _timed_region(runner, steps)
    da.qknorm_rope_attn_set_kernel_timing(False)
    kernels = da.qknorm_rope_attn_read_kernel_timing()
    ms = _timed_region(runner, steps)
    return ms, ms_events, kernels


def roofline_for(name, kernels, F, B, workload, layer_bytes=None):
    total_ms, launches = kernels[name]
    avg_s = total_ms / launches / 1e3
    if layer_bytes and name in layer_bytes:
        achieved = layer_bytes[name] / avg_s / 1e9
        rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": achieved / PEAK_HBM_GBPS, "bytes_per_launch": layer_bytes[name]}
    elif name.startswith("prefill_attn"):
        achieved = F / avg_s / 1e12
        rf = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
              "frac": achieved / PEAK_MFMA_TFLOPS}
    elif name == "fused_step_attn":
        # One launch doing both halves: stated against HBM for the decode K/V it streams, with the MFMA share of
        # the prefill FLOP it computes at the same time beside it; their sum is the step's ideal-time fraction.
        achieved = B / avg_s / 1e9
        rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": achieved / PEAK_HBM_GBPS,
              "mfma_share": {"achieved": F / avg_s / 1e12, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                             "frac": F / avg_s / 1e12 / PEAK_MFMA_TFLOPS},
              "combined_frac": achieved / PEAK_HBM_GBPS + F / avg_s / 1e12 / PEAK_MFMA_TFLOPS}
    elif name == "decode_attn_split":
        achieved = B / avg_s / 1e9
        rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": achieved / PEAK_HBM_GBPS}
    else:
        return None
    rf["kernel"] = name
    rf["avg_launch_ms"] = total_ms / launches
    rf["traffic"] = measured_traffic(name, workload)
    return rf


def cpu_baseline(w, F_total, B_total, budget_s: float = 20.0):
    """The oracle, as it stands, on a bounded sample of the same workload, scaled to the step."""
    import numpy as np

    import oracle

    threads = None
    blas = None
    try:
        from threadpoolctl import threadpool_info

        pools = threadpool_info()
        threads = max((i.get("num_threads") or 0) for i in pools) or None
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in pools if i.get("user_api") == "blas")
    except Exception:  # threadpoolctl missing or no BLAS pools
        threads = None
    cores = threads or len(os.sched_getaffinity(0))

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    t_total = 0.0
    parts = []
    if w.prefill is not None and F_total > 0:
        p = w.prefill
        h = p.heads
        lo, hi = int(p.cu_seqlens[0]), int(p.cu_seqlens[1])
        t0 = time.perf_counter()
        qt, kt, v = oracle.qk_norm_rope(f64(p.qkv[lo:hi]), f64(p.q_norm_weight), f64(p.k_norm_weight),
                                        p.positions[lo:hi].cpu().numpy(), h.num_q_heads, h.num_kv_heads,
                                        h.head_dim, h.rms_eps, h.rope_base)
        g = h.num_q_heads // h.num_kv_heads
        oracle.causal_gqa_attention(qt[:, :g], kt[:, :1], v[:, :1])
        dt = time.perf_counter() - t0
        T = hi - lo
        f_sample = 2.0 * h.head_dim * g * T * (T + 1)
        t_total += dt * F_total / f_sample
        parts.append(f"prefill: request 0 ({T} tokens), KV head 0 and its {g} query heads, {dt:.1f} s")
    if w.decode is not None and B_total > 0:
        d = w.decode
        h = d.heads
        lens = d.cache_lens.cpu().tolist()
        order = sorted(range(len(lens)), key=lambda b: lens[b])
        subset = order[len(order) // 2: len(order) // 2 + 4]
        import torch

        idx = torch.tensor(subset, device=d.k_cache.device)
        top = max(lens[b] for b in subset) + 1
        kc = f64(d.k_cache.index_select(0, idx)[:, :, :top])
        vc = f64(d.v_cache.index_select(0, idx)[:, :, :top])
        t0 = time.perf_counter()
        oracle.decode(f64(d.qkv.index_select(0, idx)), f64(d.q_norm_weight), f64(d.k_norm_weight),
                      np.array(lens)[subset], np.array(lens)[subset], kc, vc, h.num_q_heads, h.num_kv_heads,
                      h.head_dim, h.rms_eps, h.rope_base)
        dt = time.perf_counter() - t0
        b_sample = decode_kv_bytes([lens[b] for b in subset], h.num_kv_heads, h.head_dim, d.qkv.element_size())
        t_total += dt * B_total / b_sample
        parts.append(f"decode: 4 median-length requests ({[lens[b] for b in subset]} cached), all heads, {dt:.1f} s")
    value = 100.0 * (F_total / (PEAK_MFMA_TFLOPS * 1e12) + B_total / (PEAK_HBM_GBPS * 1e9)) / t_total
    return {"value": value, "unit": "% of MI355X peak", "cores": cores, "kind": "oracle",
            "numpy": np.__version__, "blas": blas or None,
            "sample": "; ".join(parts) + f"; scaled linearly to the whole step: {t_total:.1f} s per step",
            "step_seconds_est": t_total}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed_qwen3_8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the long-prefill and decode-only side runs")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this attention path runs on one GPU "
              "(each GPU would take its own share of KV heads or requests, with no exchange).", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: launched with WORLD_SIZE > 1; this benchmark runs on one GPU only.", file=sys.stderr)
        return 2

    import torch

    import decoder_attention_amd as da
    from workloads import build_workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    da.lib()
    dev = "cuda:0"

    def measure(name, steps, warmup, fused=False):
        w = build_workload(name, device=dev, parity=False)
        runner = Runner(w, torch, da, fused)
        ms, ms_events, kernels = time_steps(runner, steps, warmup)
        F, B = runner.work()
        return w, runner, ms, ms_events, kernels, F, B

    # The step as the library runs it best: a workload with both a prefill and a decode batch goes through
    # qknorm_rope_attn_mixed_step.  The same step as two calls (prefill, then decode) is timed in the same run; its
    # per-kernel figures fill `parts`.
    w, runner, ms, ms_events, kernels, F, B = measure(args.workload, args.steps, args.warmup, fused=True)
    t = ms / 1e3
    value = 100.0 * (F / (PEAK_MFMA_TFLOPS * 1e12) + B / (PEAK_HBM_GBPS * 1e9)) / t
    per_kernel = {k: {"avg_ms": v[0] / v[1], "launches_per_step": v[1] / args.steps} for k, v in kernels.items()}
    dominant = max(kernels, key=lambda k: kernels[k][0])
    roof = roofline_for(dominant, kernels, F, B, args.workload)
    fused_kernels = kernels
    separate = None
    if w.prefill is not None and w.decode is not None:
        _, srunner, sms, _, kernels, _, _ = measure(args.workload, args.steps, args.warmup, fused=False)
        separate = {"ms_per_step": sms, "value": 100.0 * (F / (PEAK_MFMA_TFLOPS * 1e12) + B / (PEAK_HBM_GBPS * 1e9))
                    / (sms / 1e3), "kernels": {k: {"avg_ms": v[0] / v[1]} for k, v in kernels.items()}}
        del srunner
    side = {}
    if separate is not None:
        side["separate_calls"] = separate
    pre_ms = sum(kernels[k][0] for k in ("qknorm_rope_kv_prefill",) + PREFILL_KERNELS if k in kernels)
    dec_ms = sum(kernels[k][0] for k in ("qknorm_rope_kv_decode", "decode_attn_split", "decode_attn_combine")
                 if k in kernels)
    if F:
        tf = F / (pre_ms / args.steps / 1e3) / 1e12
        side["prefill_call"] = {"tflops": tf, "frac_of_mfma_peak": tf / PEAK_MFMA_TFLOPS,
                                "ms": pre_ms / args.steps, "flops": F}
        side["prefill_kernel"] = prefill_roofline(kernels, F, B, args.workload)
    if B:
        gbps = B / (dec_ms / args.steps / 1e3) / 1e9
        d = w.decode
        h = d.heads
        e = d.qkv.element_size()
        # Everything the call must move: K/V read, plus the qkv rows, both norm weights, the new K/V
        # entries and the output.
        total = B + d.num_seqs * h.head_dim * e * ((h.num_q_heads + 2 * h.num_kv_heads) + 2 * h.num_kv_heads
                                                   + h.num_q_heads) + 2 * h.head_dim * e
        side["decode_call"] = {"gbps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS, "ms": dec_ms / args.steps,
                               "kv_bytes": B, "total_algorithmic_bytes": total}
        side["decode_kernel"] = roofline_for("decode_attn_split", kernels, F, B, args.workload)

    if w.prefill is not None and "qknorm_rope_kv_prefill" in kernels:
        # Kernel 1's own roofline.  bf16: the K and V columns read once and written once to the cache,
        # plus each token's fp32 cos/sin pairs (Q is rotated inside the attention kernel); fp32: every
        # qkv element read once and written once (q~, k~, v).
        p = w.prefill
        h = p.heads
        e = p.qkv.element_size()
        if e == 2:
            k1 = 2.0 * p.num_tokens * 2 * h.num_kv_heads * h.head_dim * e + p.num_tokens * h.head_dim * 4.0
        else:
            k1 = 2.0 * p.num_tokens * (h.num_q_heads + 2 * h.num_kv_heads) * h.head_dim * e
        side["kernel1_prefill"] = roofline_for("qknorm_rope_kv_prefill", kernels, F, B, args.workload,
                                               {"qknorm_rope_kv_prefill": k1})

    # Single steps, warm and after a 1 GiB read that leaves none of their data in the last-level cache.
    side["last_level_cache"] = cache_effect(runner)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, F, B)
    del runner, w
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        for name, steps in (("long_prefill_32k", 5), ("qwen3_4b_decode64", 20), ("chunked_qwen3_8b", 10)):
            ew, er, ems, _, ek, eF, eB = measure(name, steps, 2)
            rf = prefill_roofline(ek, eF, eB, name) if eF else roofline_for("decode_attn_split", ek, eF, eB, name)
            extra[name] = {"ms_per_call": ems, "kernel": rf,
                           "call_rate": (eF / (ems / 1e3) / 1e12) if eF else (eB / (ems / 1e3) / 1e9),
                           "call_rate_unit": "TFLOP/s" if eF else "GB/s"}
            if not eF:  # decode: the same call with nothing of its K/V left in the last-level cache
                ce = cache_effect(er)
                ce["call_rate_after_1gib_read"] = eB / (ce["ms_single_step_after_1gib_read"] / 1e3) / 1e9
                extra[name]["last_level_cache"] = ce
            del er, ew
            torch.cuda.empty_cache()
        # Steps next to the attention layer, each against the HBM roofline.
        for name, steps in (("residual_rmsnorm_qwen3_8b", 20), ("next_token_qwen3_8b", 20)):
            ew, er, ems, _, ek, _, _ = measure(name, steps, 2)
            lb = er.hbm_bytes()
            extra[name] = {"ms_per_call": ems,
                           "kernels": {k: roofline_for(k, ek, 0.0, 0.0, name, lb) for k in lb if k in ek}}
            del er, ew
            torch.cuda.empty_cache()

    record = {
        "metric": "prefill attention TFLOP/s + decode KV GB/s, as % of MI355X peak",
        "value": value,
        "unit": "% of MI355X peak",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_with_kernel_events": ms_events,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal qkv, norm weights 1+0.1N, cache contents N(0,1))",
        "config": {"workload": args.workload, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                   "prefill_seqlens": [4096] * 4 if args.workload == "mixed_qwen3_8b" else None,
                   "decode_requests": 128 if args.workload == "mixed_qwen3_8b" else None,
                   "decode_cache_lens": "U[1,16384], seed 1005" if args.workload == "mixed_qwen3_8b" else None,
                   "prefill_flops": F, "decode_kv_bytes": B},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parts": side,
        "kernels": per_kernel,
        "side_workloads": extra,
    }
    print(json.dumps(record), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
