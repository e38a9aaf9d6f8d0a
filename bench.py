#!/usr/bin/env python3
"""Throughput of QK-norm + RoPE + causal GQA attention on one MI355X.

A step is one pass of the whole attention hot path over one batch: the
default workload is the mixed packed step on Qwen3-8B-shaped heads (Hq=32,
Hkv=8, D=128): a prefill of 4 requests x 4096 tokens (QK-norm + RoPE +
K/V-cache write + causal attention) and one decode step for 128 requests whose
caches hold U[1, 16384] entries, run through qknorm_rope_attn_mixed_step.

Metric: attention work as a fraction of the MI355X roofline.  For a step,
    value = 100 * (F / P_mfma + B / P_hbm) / t_step
with F the causal prefill FLOPs (sum over requests of 2*D*Hq*T(T+1)), B the
decode K/V bytes (sum over requests of 2*Hkv*(L+1)*D*2), P_mfma = 2500 TFLOP/s
(dense bf16 MFMA) and P_hbm = 8000 GB/s; i.e. the ideal time of the step's
work on each roofline divided by the measured step time.  Inputs are resident
in HBM before timing starts.

Timing: after W warm-up steps, K steps each bracketed by their own HIP events;
t_step is their median (p10 and p90 beside it).  In the same K steps the step's
dominant kernel is timed by events attached to its own dispatch (no other
kernel is timed there), so its duration and the step time come from one region.
The same is repeated with a 1 GiB read before each step, which leaves nothing of
the step's data in the 256 MB last-level cache ("flushed").  The other configs
(the pages' 12-token run, the 64-token layer, the varlen prefill, the 64-request
decode, the 32k prefill, the two-call step, the chunked append, the paged
decodes, the layer steps beside attention) and a roofline calibration
(streaming read, MFMA loop) follow as side workloads.

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


def spread(times):
    """(median, p10, p90) of a list of times."""
    t = sorted(times)
    n = len(t)
    return t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2]), t[(n - 1) // 10], t[((n - 1) * 9) // 10]


def weight_bound(q_norm_weight, k_norm_weight) -> float:
    """max|w_q| * max|w_k|: fixed for a layer, so a caller computes it once (qkra_config.qk_weight_bound)."""
    return float(q_norm_weight.float().abs().max()) * float(k_norm_weight.float().abs().max())


class Runner:
    """Holds device inputs/outputs/workspaces of a workload and issues its calls (one step = every call)."""

    def __init__(self, w, torch, da, fused: bool = False, paged_page_size: int = 0, use_bound: bool = True):
        self.torch, self.da, self.w = torch, da, w
        self.calls = []
        if w.prefill is not None:
            p = w.prefill
            h = p.heads
            bound = weight_bound(p.q_norm_weight, p.k_norm_weight) if use_bound else 0.0
            cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, p.qkv.dtype, h.rms_eps, h.rope_base,
                                 qk_weight_bound=bound)
            out = torch.empty((p.num_tokens, h.num_q_heads * h.head_dim), dtype=p.qkv.dtype, device=p.qkv.device)
            ws_bytes = da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_PREFILL, p.num_tokens, p.max_seqlen)
            ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=p.qkv.device)
            args = (cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens, p.num_tokens,
                    p.num_seqs, p.max_seqlen, p.k_cache, p.v_cache, p.cache_capacity, out, ws, ws_bytes)
            self.calls.append(("prefill", da.qknorm_rope_attn_prefill, args, (out, ws)))
            for s, row in enumerate(w.chained_decode_qkv):  # decode steps on the prefill's own caches
                lens = torch.full((p.num_seqs,), p.seqlens[0] + s, dtype=torch.int32, device=p.qkv.device)
                dout = torch.empty((p.num_seqs, h.num_q_heads * h.head_dim), dtype=p.qkv.dtype, device=p.qkv.device)
                dws_bytes = da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_DECODE, p.num_seqs,
                                                                p.seqlens[0] + s)
                dws = torch.empty((dws_bytes,), dtype=torch.uint8, device=p.qkv.device)
                args = (cfg, row, p.q_norm_weight, p.k_norm_weight, lens, lens, p.num_seqs, p.seqlens[0] + s,
                        p.k_cache, p.v_cache, p.cache_capacity, dout, dws, dws_bytes)
                self.calls.append((f"decode_step_{s}", da.qknorm_rope_attn_decode, args, (lens, dout, dws)))
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
            self.calls.append(("append", da.qknorm_rope_attn_prefill_append, args, (out, ws)))
        if w.decode is not None:
            d = w.decode
            h = d.heads
            cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, d.qkv.dtype, h.rms_eps, h.rope_base)
            out = torch.empty((d.num_seqs, h.num_q_heads * h.head_dim), dtype=d.qkv.dtype, device=d.qkv.device)
            ws_bytes = da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_DECODE, d.num_seqs, d.max_cache_len)
            ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=d.qkv.device)
            if paged_page_size:
                from workloads import paged_from_contiguous

                pc = paged_from_contiguous(d.k_cache, d.v_cache, paged_page_size, seed=4242, parity=False)
                d.k_cache = d.v_cache = None  # the pool holds the cache now
                desc = da.make_paged_cache(pc.k_pool, pc.v_pool, pc.block_table, pc.num_pages, pc.page_size,
                                           pc.pages_per_seq)
                args = (cfg, d.qkv, d.q_norm_weight, d.k_norm_weight, d.positions, d.cache_lens, d.num_seqs,
                        d.max_cache_len, desc, out, ws, ws_bytes)
                self.calls.append(("decode_paged", da.qknorm_rope_attn_decode_paged, args, (out, ws, pc, desc)))
            else:
                args = (cfg, d.qkv, d.q_norm_weight, d.k_norm_weight, d.positions, d.cache_lens, d.num_seqs,
                        d.max_cache_len, d.k_cache, d.v_cache, d.cache_capacity, out, ws, ws_bytes)
                self.calls.append(("decode", da.qknorm_rope_attn_decode, args, (out, ws)))
        if w.norm is not None:
            n = w.norm
            out = torch.empty_like(n.x)
            res = n.residual if n.has_residual else torch.empty_like(n.x)
            args = (da_dtype(da, n.x), n.rms_eps, n.x, res, n.has_residual, n.weight, out, n.x.shape[0],
                    n.x.shape[1])
            self.calls.append(("fused_add_rmsnorm", da.qknorm_rope_attn_fused_add_rmsnorm, args, (out, res)))
        if w.next_token is not None:
            nt = w.next_token
            b, c, v = len(nt.seqlens), nt.hidden.shape[1], nt.logits.shape[1]
            last = torch.empty((b, c), dtype=nt.hidden.dtype, device=nt.hidden.device)
            args = (da_dtype(da, nt.hidden), nt.hidden, nt.cu_seqlens, nt.hidden.shape[0], b, c, last)
            self.calls.append(("gather_last", da.qknorm_rope_attn_gather_last, args, (last,)))
            idx = torch.empty((b,), dtype=torch.int32, device=nt.logits.device)
            ws_bytes = da.qknorm_rope_attn_argmax_workspace_bytes(b, v)
            ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=nt.logits.device)
            args = (da_dtype(da, nt.logits), nt.logits, b, v, nt.logits.stride(0), idx, ws, ws_bytes)
            self.calls.append(("argmax", da.qknorm_rope_attn_argmax, args, (idx, ws)))

        if fused and w.prefill is not None and w.decode is not None and not w.chained_decode_qkv:
            # The same step through qknorm_rope_attn_mixed_step: one call, the prefill attention and the decode
            # split in one launch (both halves share the norm weights, as one layer's do).
            (_, _, pa, pkeep), (_, _, dargs, dkeep) = self.calls[0], self.calls[1]
            mixed = (pa[0], pa[2], pa[3]) + pa[1:2] + pa[4:] + dargs[1:2] + dargs[4:]
            self.calls = [("mixed_step", da.qknorm_rope_attn_mixed_step, mixed, pkeep + dkeep)] + self.calls[2:]

    def step(self):
        for _, fn, args, _ in self.calls:
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


def kernel_ids(da):
    names = {}
    for k in range(32):
        n = da.qknorm_rope_attn_kernel_name(k)
        if n == "unknown":
            break
        names[n] = k
    return names


def timed_reps(runner, reps: int, warmup: int, mask: int, evict: bool = False, per_call: bool = False):
    """`warmup` steps, then `reps` steps each between its own events (per call with `per_call`), with the
    kernels in `mask` timed on their own dispatches over the same steps.  With `evict`, a 1 GiB read (outside
    the events) precedes every step.  Returns (step times in ms, {call: times} or None, kernel table)."""
    torch, da = runner.torch, runner.da
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if evict else None
    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    da.qknorm_rope_attn_read_kernel_timing()  # drop anything recorded before
    da.qknorm_rope_attn_set_kernel_timing(mask)
    steps, calls = [], []
    for _ in range(reps):
        if evict:
            scratch.sum()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(runner.calls) + 1 if per_call else 2)]
        ev[0].record()
        for i, (_, fn, args, _) in enumerate(runner.calls):
            status = fn(*args)
            if status != 0:
                raise da.QkraError(status, fn.__name__)
            if per_call:
                ev[i + 1].record()
        if not per_call:
            ev[1].record()
        steps.append(ev)
    torch.cuda.synchronize()
    da.qknorm_rope_attn_set_kernel_timing(0)
    kernels = da.qknorm_rope_attn_read_kernel_timing()
    times = [ev[0].elapsed_time(ev[-1]) for ev in steps]
    per = None
    if per_call:
        per = {name: [ev[i].elapsed_time(ev[i + 1]) for ev in steps] for i, (name, _, _, _) in enumerate(runner.calls)}
    del scratch
    return times, per, kernels


WRITES_AS_MUCH_AS_READS = {"qknorm_rope_kv_prefill", "fused_add_rmsnorm"}


def roofline_for(name, kernels, F, B, workload, layer_bytes=None, measured=None):
    """The roofline object of kernel `name` from its timed launches."""
    if name not in kernels:
        return None
    total_ms, launches = kernels[name]
    avg_s = total_ms / launches / 1e3
    if layer_bytes and name in layer_bytes:
        achieved = layer_bytes[name] / avg_s / 1e9
        rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": achieved / PEAK_HBM_GBPS, "bytes_per_launch": layer_bytes[name]}
    elif name.startswith("prefill_attn"):
        achieved = F / avg_s / 1e12
        rf = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
              "frac": achieved / PEAK_MFMA_TFLOPS, "flop_per_launch": F}
    elif name == "fused_step_attn":
        # One launch doing both halves: stated against HBM for the decode K/V it streams, with the MFMA share of
        # the prefill FLOP it computes at the same time beside it.  Their sum is the ideal serial time over the
        # kernel's time, not a roofline fraction: the two halves overlap in the launch.
        achieved = B / avg_s / 1e9
        rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": achieved / PEAK_HBM_GBPS, "bytes_per_launch": B,
              "mfma_share": {"achieved": F / avg_s / 1e12, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                             "frac": F / avg_s / 1e12 / PEAK_MFMA_TFLOPS, "flop_per_launch": F},
              "serial_ideal_over_kernel": achieved / PEAK_HBM_GBPS + F / avg_s / 1e12 / PEAK_MFMA_TFLOPS}
    elif name == "decode_attn_split":
        achieved = B / avg_s / 1e9
        rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": achieved / PEAK_HBM_GBPS, "bytes_per_launch": B}
    else:
        return None
    rf["kernel"] = name
    rf["avg_launch_ms"] = total_ms / launches
    rf["launches"] = launches
    rf["traffic"] = measured_traffic(name, workload)
    if measured:
        # Kernels that write about as many bytes as they read are set against the copy, the rest against the
        # streaming read or the MFMA loop.
        kind = ("stream_copy" if name in WRITES_AS_MUCH_AS_READS else "stream_read") if rf["unit"] == "GB/s" \
            else "mfma_loop"
        m = measured.get({"stream_copy": "copy_gbps", "stream_read": "hbm_gbps", "mfma_loop": "mfma_tflops"}[kind])
        if m:
            rf["frac_of_measured_peak"] = rf["achieved"] / m
            rf["measured_peak"] = kind
    return rf


def calibration(torch, da):
    """What this part sustains: a 4 GiB streaming read, a 2 GiB copy and a bf16 MFMA loop (median of 10 launches each)."""
    dev = "cuda"
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1024, dtype=torch.float32, device=dev)

    def med(fn, n=10):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return spread(ts)[0]

    reads = {}
    for wg in (512, 1024, 2048):  # 8, 16 and 32 wavefronts per CU; the best is the part's streaming rate
        reads[wg] = med(lambda: da.check(da.qkra_calibrate_stream_read(buf, nbytes, sink, wg), "stream_read"))
    wg_read = min(reads, key=reads.get)
    t_read = reads[wg_read]
    half = nbytes // 2  # copy the first 2 GiB of the buffer onto the second
    src, dst = buf[: half // 4], buf[half // 4:]
    t_copy = med(lambda: da.check(da.qkra_calibrate_stream_copy(src, dst, half), "stream_copy"))
    del src, dst
    iters, wg_mfma = 2000, 512
    t_mfma = med(lambda: da.check(da.qkra_calibrate_mfma_bf16(iters, sink, wg_mfma), "mfma_loop"))
    flop = da.qkra_calibrate_mfma_flop(iters, wg_mfma)
    del buf
    return {"hbm_gbps": nbytes / (t_read / 1e3) / 1e9, "mfma_tflops": flop / (t_mfma / 1e3) / 1e12,
            "stream_read": f"4 GiB, each wavefront a contiguous share, 16-byte non-temporal loads, 8 in flight; "
                           f"best of 512/1024/2048 workgroups of 256 ({wg_read}), median of 10",
            "stream_read_gbps_by_workgroups": {str(k): nbytes / (v / 1e3) / 1e9 for k, v in reads.items()},
            "copy_gbps": 2 * half / (t_copy / 1e3) / 1e9,
            "stream_copy": "2 GiB onto 2 GiB, one 16-byte piece per thread with non-temporal loads and stores; read "
                           "plus written bytes over the time, median of 10",
            "mfma_loop": f"{iters} rounds of 4 independent v_mfma_f32_32x32x16_bf16 per wavefront, "
                         f"{wg_mfma} workgroups of 4 wavefronts, median of 10"}


def same_size_copy(torch, da, total_bytes, reps=20, batch=10):
    """GB/s (read plus written) of the calibration copy moving `total_bytes` in all (half read, half written):
    the ceiling of a kernel of that size that writes as much as it reads, its ramp and tail included.  Each
    sample times `batch` copies launched back to back between two events (so the launch itself is hidden,
    as for a kernel inside a step); the median of `reps` samples.  None without the calibration library."""
    half = int(total_bytes // 2) // 16 * 16
    if half <= 0:
        return None
    src = torch.empty(half // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    try:
        run = lambda: da.check(da.qkra_calibrate_stream_copy(src, dst, half), "stream_copy")  # noqa: E731
        run()
    except RuntimeError:
        return None
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(batch):
            run()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / batch)
    del src, dst
    return 2 * half / (spread(ts)[0] / 1e3) / 1e9


def with_same_size_copy(rf, gbps):
    """Adds the same-size copy's rate to a roofline object that is set against the copy."""
    if rf is not None and gbps:
        rf["same_size_copy_gbps"] = gbps
        rf["frac_of_same_size_copy"] = rf["achieved"] / gbps
    return rf


def cpu_baseline(w, F_total, B_total):
    """The oracle, as it stands, on the host: the whole decode half at full size, and one (request, KV head)
    group of the prefill scaled by FLOP (the groups are independent and cost the same)."""
    import numpy as np
    import torch

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
    cores = len(os.sched_getaffinity(0))

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    t_total = 0.0
    parts = []
    if w.prefill is not None and F_total > 0:
        p = w.prefill
        h = p.heads
        lo, hi = int(p.cu_seqlens[0]), int(p.cu_seqlens[1])
        qkv, wq, wk, pos = f64(p.qkv[lo:hi]), f64(p.q_norm_weight), f64(p.k_norm_weight), p.positions[lo:hi].cpu().numpy()
        t0 = time.perf_counter()
        qt, kt, v = oracle.qk_norm_rope(qkv, wq, wk, pos, h.num_q_heads, h.num_kv_heads, h.head_dim, h.rms_eps,
                                        h.rope_base)
        g = h.num_q_heads // h.num_kv_heads
        oracle.causal_gqa_attention(qt[:, :g], kt[:, :1], v[:, :1])
        dt = time.perf_counter() - t0
        T = hi - lo
        f_sample = 2.0 * h.head_dim * g * T * (T + 1)
        t_total += dt * F_total / f_sample
        parts.append(f"prefill: request 0 ({T} tokens), KV head 0 and its {g} query heads in {dt:.2f} s, scaled by "
                     f"FLOP to all {F_total / f_sample:.0f} such groups")
    if w.decode is not None and B_total > 0:
        d = w.decode
        h = d.heads
        lens = d.cache_lens.cpu().tolist()
        dt = 0.0
        for c0 in range(0, len(lens), 8):  # every request; inputs widened to fp64 outside the timed calls
            sub = list(range(c0, min(c0 + 8, len(lens))))
            idx = torch.tensor(sub, device=d.k_cache.device)
            top = max(lens[b] for b in sub) + 1
            args = (f64(d.qkv.index_select(0, idx)), f64(d.q_norm_weight), f64(d.k_norm_weight),
                    np.array(lens)[sub], np.array(lens)[sub], f64(d.k_cache.index_select(0, idx)[:, :, :top]),
                    f64(d.v_cache.index_select(0, idx)[:, :, :top]))
            t0 = time.perf_counter()
            oracle.decode(*args, h.num_q_heads, h.num_kv_heads, h.head_dim, h.rms_eps, h.rope_base)
            dt += time.perf_counter() - t0
            del args
        t_total += dt
        parts.append(f"decode: all {len(lens)} requests at full size, {dt:.2f} s")
    value = 100.0 * (F_total / (PEAK_MFMA_TFLOPS * 1e12) + B_total / (PEAK_HBM_GBPS * 1e9)) / t_total
    return {"value": value, "unit": "% of MI355X peak", "cores": threads or cores, "affinity_cores": cores,
            "blas_threads": threads, "kind": "oracle", "numpy": np.__version__, "blas": blas or None,
            "sample": "; ".join(parts) + f"; {t_total:.1f} s per step", "step_seconds": t_total}


def oracle_host_seconds(w, F_total, B_total, sample_rows=0):
    """The oracle's host time for one call of a side workload: as cpu_baseline times it, or, for a prefill too
    long for that (one KV head over 32k tokens), Q/K-norm + RoPE of every token and `sample_rows` output rows
    spread over the request (all heads each), scaled by the causal FLOP of the sampled rows."""
    if not sample_rows or w.prefill is None:
        b = cpu_baseline(w, F_total, B_total)
        return {"seconds": b["step_seconds"], "sample": b["sample"], "cores": b["cores"]}
    import numpy as np

    import oracle

    p = w.prefill
    h = p.heads
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    qkv, wq, wk, pos = f64(p.qkv), f64(p.q_norm_weight), f64(p.k_norm_weight), p.positions.cpu().numpy()
    cu = p.cu_seqlens.cpu().tolist()
    t0 = time.perf_counter()
    qt, kt, v = oracle.qk_norm_rope(qkv, wq, wk, pos, h.num_q_heads, h.num_kv_heads, h.head_dim, h.rms_eps,
                                    h.rope_base)
    t_norm = time.perf_counter() - t0
    lo, hi = cu[0], cu[1]
    rows = sorted(set(int(x) for x in np.linspace(lo, hi - 1, sample_rows)))
    t0 = time.perf_counter()
    oracle.prefill_rows(qt, kt, v, cu, rows)
    t_rows = time.perf_counter() - t0
    f_rows = sum(4.0 * h.head_dim * h.num_q_heads * (r - lo + 1) for r in rows)
    total = t_norm + t_rows * F_total / f_rows
    return {"seconds": total, "cores": len(os.sched_getaffinity(0)),
            "sample": f"Q/K-norm + RoPE of all {p.num_tokens} tokens in {t_norm:.2f} s; {len(rows)} rows spread "
                      f"over request 0 (every head) in {t_rows:.2f} s, scaled by causal FLOP to all rows"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed_qwen3_8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the side workloads and the calibration")
    ap.add_argument("--no-weight-bound", action="store_true",
                    help="do not pass the norm weights' bound (every bf16 prefill then launches both softmax kernels)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="run a decode-only workload's decode through the paged call with this page size")
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
    ids = kernel_ids(da)
    mask_of = lambda names: sum(1 << ids[n] for n in names)  # noqa: E731

    # Roofline calibration first (its own library), so every rate below can be set against it as well.
    measured = None
    if not args.no_extra:
        try:
            measured = calibration(torch, da)
        except RuntimeError as e:  # the calibration library is not built
            measured = {"error": str(e)}
        torch.cuda.empty_cache()

    # ---- the headline: the mixed step through qknorm_rope_attn_mixed_step ----------------------------------
    w = build_workload(args.workload, device=dev, parity=False)
    use_bound = not args.no_weight_bound
    runner = Runner(w, torch, da, fused=True, paged_page_size=args.page_size if w.prefill is None else 0,
                    use_bound=use_bound)
    F, B = runner.work()
    ideal_s = F / (PEAK_MFMA_TFLOPS * 1e12) + B / (PEAK_HBM_GBPS * 1e9)
    # Every kernel timed once over a few steps (which perturbs the step) to find the dominant one ...
    probe_t, _, probe_k = timed_reps(runner, 10, 3, -1)
    dominant = max(probe_k, key=lambda k: probe_k[k][0])
    # ... then the measured steps, with only that kernel timed.
    times, _, kernels = timed_reps(runner, args.steps, args.warmup, mask_of([dominant]))
    ms, p10, p90 = spread(times)
    value = 100.0 * ideal_s / (ms / 1e3)
    roof = roofline_for(dominant, kernels, F, B, args.workload, measured=measured)
    ftimes, _, fk = timed_reps(runner, 20, 2, mask_of([dominant]), evict=True)
    fms, fp10, fp90 = spread(ftimes)
    flushed = {"ms_per_step": fms, "p10": fp10, "p90": fp90, "value": 100.0 * ideal_s / (fms / 1e3),
               "kernel_avg_ms": fk[dominant][0] / fk[dominant][1], "reps": 20,
               "protocol": "1 GiB read before each step, outside its events"}
    all_timed = {"ms_per_step_median": spread(probe_t)[0], "reps": 10,
                 "kernels": {k: {"avg_ms": v[0] / v[1], "launches_per_step": v[1] / 10} for k, v in probe_k.items()}}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, F, B)
    del runner, w
    torch.cuda.empty_cache()

    # ---- side workloads ----------------------------------------------------------------------------------
    side = {}

    def run_side(name, reps, warmup, timed_names, per_call=False, fused=False, paged=0, evict=False, keep=None):
        sw = build_workload(name, device=dev, parity=False)
        r = Runner(sw, torch, da, fused=fused, paged_page_size=paged, use_bound=use_bound)
        if keep:  # time only these calls of the workload (e.g. the decode half of the mixed step)
            r.calls = [c for c in r.calls if c[0].startswith(keep)]
            if keep == "decode":
                sw.prefill = None
        t, per, k = timed_reps(r, reps, warmup, mask_of([n for n in timed_names if n in ids]), per_call=per_call)
        out = {"ms_per_call": spread(t)[0], "p10": spread(t)[1], "p90": spread(t)[2], "reps": reps}
        if per:
            out["calls_ms"] = {c: spread(v)[0] for c, v in per.items()}
        if evict:
            te, _, _ = timed_reps(r, 20, 2, 0, evict=True)
            out["ms_per_call_flushed"] = spread(te)[0]
        return sw, r, out, k

    if not args.no_extra:
        # The pages' own run shape: prefill of 12 tokens, then 9 decode steps on its cache (latency only).
        sw, r, out, k = run_side("pages_t12_decode9", 50, 5, [], per_call=True)
        calls = out.pop("calls_ms")
        out = {"prefill_us": calls["prefill"] * 1e3,
               "decode_step_us": [calls[f"decode_step_{s}"] * 1e3 for s in range(9)],
               "chain_us": out["ms_per_call"] * 1e3, "reps": 50, "bound": "latency"}
        side["pages_t12_decode9"] = out
        del sw, r
        # The 64-token layer (Hq 4, Hkv 2, D 64): prefill, then one decode at position 64 (latency only).
        sw, r, out, k = run_side("single_t64_hq4_hkv2_d64", 50, 5, [], per_call=True)
        calls = out.pop("calls_ms")
        side["single_t64_hq4_hkv2_d64"] = {"prefill_us": calls["prefill"] * 1e3, "decode_us": calls["decode_step_0"] * 1e3,
                                          "reps": 50, "bound": "latency"}
        if not args.no_cpu_baseline:  # the oracle's prefill of the same 64 tokens on the host
            side["single_t64_hq4_hkv2_d64"]["cpu_oracle_prefill"] = oracle_host_seconds(sw, r.work()[0], 0.0)
        del sw, r
        # Prefill-only workloads against the MFMA roofline (the attention kernel timed in the same calls).
        for name, reps in (("qwen3_0p6b_prefill_varlen8", 50), ("long_prefill_32k", 12), ("chunked_qwen3_8b", 20)):
            sw, r, out, k = run_side(name, reps, 3, list(PREFILL_KERNELS))
            Fs, _ = r.work()
            kname = working_prefill_kernel(k)
            out["call_tflops"] = Fs / (out["ms_per_call"] / 1e3) / 1e12
            out["kernel"] = roofline_for(kname, k, Fs, 0.0, name, measured=measured)
            others = {n: k[n][0] / k[n][1] for n in PREFILL_KERNELS if n in k and n != kname}
            if others:
                out["kernel"]["other_path_avg_launch_ms"] = others
            if not args.no_cpu_baseline and name != "chunked_qwen3_8b":
                out["cpu_oracle"] = oracle_host_seconds(sw, Fs, 0.0, sample_rows=96 if name == "long_prefill_32k" else 0)
            side[name] = out
            del sw, r
            torch.cuda.empty_cache()
        # Decode workloads against the HBM roofline, contiguous and paged (64-slot pages), warm and flushed.
        for name, paged in (("qwen3_4b_decode64", 0), ("qwen3_4b_decode64", 64), ("mixed_qwen3_8b", 64)):
            key = name if not paged else f"{name}_decode_paged{paged}"
            sw, r, out, k = run_side(name, 50, 5, ["decode_attn_split"], paged=paged, evict=True, keep="decode")
            _, Bs = r.work()
            out["call_gbps"] = Bs / (out["ms_per_call"] / 1e3) / 1e9
            out["call_gbps_flushed"] = Bs / (out["ms_per_call_flushed"] / 1e3) / 1e9
            out["kernel"] = roofline_for("decode_attn_split", k, 0.0, Bs, key, measured=measured)
            if not args.no_cpu_baseline and key == "qwen3_4b_decode64":
                out["cpu_oracle"] = oracle_host_seconds(sw, 0.0, Bs)
            side[key] = out
            del sw, r
            torch.cuda.empty_cache()
        # The mixed step as two calls (prefill, then decode), each call timed, each attention kernel timed.
        sw, r, out, k = run_side("mixed_qwen3_8b", 50, 5, list(PREFILL_KERNELS) + ["decode_attn_split",
                                                                                   "qknorm_rope_kv_prefill"],
                                 per_call=True)
        Fs, Bs = r.work()
        calls = out.pop("calls_ms")
        kname = working_prefill_kernel(k)
        p = sw.prefill
        h = p.heads
        k1_bytes = 2.0 * p.num_tokens * 2 * h.num_kv_heads * h.head_dim * 2 + p.num_tokens * h.head_dim * 4.0
        side["mixed_qwen3_8b_two_calls"] = {
            "ms_per_step": out["ms_per_call"], "p10": out["p10"], "p90": out["p90"],
            "value": 100.0 * ideal_s / (out["ms_per_call"] / 1e3),
            "prefill_call_ms": calls["prefill"], "decode_call_ms": calls["decode"],
            "prefill_call_tflops": Fs / (calls["prefill"] / 1e3) / 1e12,
            "decode_call_gbps": Bs / (calls["decode"] / 1e3) / 1e9,
            "prefill_kernel": roofline_for(kname, k, Fs, Bs, "mixed_qwen3_8b", measured=measured),
            "decode_kernel": roofline_for("decode_attn_split", k, Fs, Bs, "mixed_qwen3_8b", measured=measured),
            "kernel1_prefill": with_same_size_copy(
                roofline_for("qknorm_rope_kv_prefill", k, Fs, Bs, "mixed_qwen3_8b",
                             {"qknorm_rope_kv_prefill": k1_bytes}, measured=measured),
                same_size_copy(torch, da, k1_bytes))}
        del sw, r
        torch.cuda.empty_cache()
        # Steps next to the attention layer: the fused add + RMSNorm against HBM; the last-row gather and the
        # argmax are latency rows (a few microseconds each).
        for name in ("residual_rmsnorm_qwen3_8b", "next_token_qwen3_8b"):
            sw = build_workload(name, device=dev, parity=False)
            r = Runner(sw, torch, da)
            lb = r.hbm_bytes()
            t, per, k = timed_reps(r, 50, 5, mask_of([n for n in lb if n in ids]), per_call=True)
            entry = {"calls_us": {c: spread(v)[0] * 1e3 for c, v in per.items()}, "reps": 50}
            if "fused_add_rmsnorm" in lb:
                entry["kernel"] = with_same_size_copy(
                    roofline_for("fused_add_rmsnorm", k, 0.0, 0.0, name, lb, measured=measured),
                    same_size_copy(torch, da, lb["fused_add_rmsnorm"]))
            else:
                entry["bound"] = "latency"
            side[name] = entry
            del sw, r
            torch.cuda.empty_cache()

    record = {
        "metric": "prefill attention TFLOP/s + decode KV GB/s, as % of MI355X peak",
        "value": value,
        "unit": "% of MI355X peak",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_p10": p10,
        "ms_per_step_p90": p90,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal qkv, norm weights 1+0.1N, cache contents N(0,1))",
        "qk_weight_bound_passed": use_bound,
        "config": {"workload": args.workload, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                   "prefill_seqlens": [4096] * 4 if args.workload == "mixed_qwen3_8b" else None,
                   "decode_requests": 128 if args.workload == "mixed_qwen3_8b" else None,
                   "decode_cache_lens": "U[1,16384], seed 1005" if args.workload == "mixed_qwen3_8b" else None,
                   "prefill_flops": F, "decode_kv_bytes": B},
        "roofline": roof,
        "cpu_baseline": cpu,
        "flushed": flushed,
        "kernels_all_timed": all_timed,
        "calibration": measured,
        "side_workloads": side,
    }
    print(json.dumps(record), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
