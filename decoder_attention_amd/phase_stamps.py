"""Per-workgroup phase times of the bf16 prefill attention kernel.

Runs one prefill (or chunk-append) workload, or the mixed step of a workload
with both halves (its prefill and decode in the fused kernel), through the profiling build of the
library (libqknorm_rope_attn_stamps.so, include/qkra_phase_stamps.h), whose
prefill kernels stamp the 100 MHz constant clock at fixed points of every
workgroup's life, and prints where the time goes: per work item (prologue,
first step, later steps, epilogue) and per CU (prologue, tile loop, epilogue,
gaps between one workgroup's end and the next one's start, idle tail); for the
mixed step also when the decode-role and prefill-role workgroups ran.

    python -m decoder_attention_amd.phase_stamps --workload prefill_4x4096_qwen3_8b

The workload is generated on the GPU from the seeded recipe in ``workloads``;
the stamped call is the last of a warm-up of about half a second of the same
call, with the records cleared before it.  Build the profiling library first
(``python decoder_attention_amd/build.py``).
"""

from __future__ import annotations

import argparse
import collections
import json
import os
import sys
import time

import numpy as np

from .build import STAMPS_LIB_PATH

TICK_US = 0.01  # s_memrealtime counts a 100 MHz clock


def _load(path=STAMPS_LIB_PATH):
    import decoder_attention_amd as da

    da.select_library(path)
    da.lib()
    return da


def _prefill_call(da, torch, w, use_bound: bool):
    """A closure that issues the workload's prefill (or append) call once."""
    if w.prefill is not None:
        p = w.prefill
        h = p.heads
        bound = (float(p.q_norm_weight.float().abs().max()) * float(p.k_norm_weight.float().abs().max())
                 if use_bound else 0.0)
        cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, p.qkv.dtype, h.rms_eps, h.rope_base,
                             qk_weight_bound=bound)
        out, ws = da.prefill(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens,
                             p.max_seqlen, p.k_cache, p.v_cache)

        def call():
            da.prefill(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens, p.max_seqlen,
                       p.k_cache, p.v_cache, out=out, workspace=ws)
        return call, h, p.seqlens, [0] * len(p.seqlens)
    a = w.append
    if a is None:
        raise SystemExit(f"workload {w.name} has no prefill or append call")
    h = a.heads
    cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, a.qkv.dtype, h.rms_eps, h.rope_base)
    out, ws = da.prefill_append(cfg, a.qkv, a.q_norm_weight, a.k_norm_weight, a.positions, a.cu_seqlens,
                                a.cache_lens, a.max_seqlen, a.max_cache_len, a.k_cache, a.v_cache)

    def call():
        # The append writes its chunk behind each request's history; rewriting the same slots each time is
        # the same work, so the caches are not restored between calls.
        da.prefill_append(cfg, a.qkv, a.q_norm_weight, a.k_norm_weight, a.positions, a.cu_seqlens, a.cache_lens,
                          a.max_seqlen, a.max_cache_len, a.k_cache, a.v_cache, out=out, workspace=ws)
    return call, h, a.seqlens, a.past_lens


def _mixed_call(da, torch, w):
    """A closure that issues the workload's mixed step (prefill and decode in one fused launch) once."""
    p, d = w.prefill, w.decode
    h = p.heads
    bound = float(p.q_norm_weight.float().abs().max()) * float(p.k_norm_weight.float().abs().max())
    cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, p.qkv.dtype, h.rms_eps, h.rope_base,
                         qk_weight_bound=bound)
    po, do, pws, dws = da.mixed_step(cfg, p.q_norm_weight, p.k_norm_weight, p.qkv, p.positions, p.cu_seqlens,
                                     p.max_seqlen, p.k_cache, p.v_cache, d.qkv, d.positions, d.cache_lens,
                                     d.max_cache_len, d.k_cache, d.v_cache)

    def call():
        da.mixed_step(cfg, p.q_norm_weight, p.k_norm_weight, p.qkv, p.positions, p.cu_seqlens, p.max_seqlen,
                      p.k_cache, p.v_cache, d.qkv, d.positions, d.cache_lens, d.max_cache_len, d.k_cache, d.v_cache,
                      prefill_out=po, prefill_workspace=pws, decode_out=do, decode_workspace=dws)
    return call


def summarize(rec: np.ndarray) -> dict:
    """rec: uint64 [workgroups, waves, slots] as the profiling build writes it."""
    from types import SimpleNamespace

    S = SimpleNamespace(ENTRY=0, ISSUED=1, Q_READY=2, LOOP=3, FIRST_STEP=4, LOOP_END=5, END=6, WHERE=7)
    r = rec.astype(np.int64)
    ran = (r[:, :, S.END] > 0).all(axis=1) & (r[:, 0, S.WHERE] >= 0)  # bit 63: the fused step's decode role
    r = r[ran]
    if r.shape[0] == 0:
        raise SystemExit("no workgroup of the prefill kernel ran a work item")
    where = r[:, 0, S.WHERE]
    hw, xcc = where & 0xFFFF, (where >> 16) & 0xF
    ntiles = (where >> 20) & 0xFFFF
    cu = (xcc << 8) | ((hw >> 8) & 0xFF)  # XCC, shader engine, shader array, CU
    t = lambda k: r[:, :, k] * TICK_US  # noqa: E731  (per wavefront, microseconds)
    wg_start = t(S.ENTRY).min(1)
    wg_end = t(S.END).max(1)
    base, span = wg_start.min(), wg_end.max() - wg_start.min()

    def mean_p(x):
        return {"mean": float(np.mean(x)), "p10": float(np.percentile(x, 10)), "p90": float(np.percentile(x, 90))}

    d = lambda a, b: (t(b) - t(a)).mean(1)  # noqa: E731  (per workgroup: mean over its wavefronts)
    steps = ntiles.astype(np.float64)
    later = d(S.FIRST_STEP, S.LOOP_END)
    multi = steps > 1
    item = {
        "issue_loads": mean_p(d(S.ENTRY, S.ISSUED)),
        "q_normalise_rotate": mean_p(d(S.ISSUED, S.Q_READY)),
        "tile0_to_loop": mean_p(d(S.Q_READY, S.LOOP)),
        "prologue": mean_p(d(S.ENTRY, S.LOOP)),
        "first_step": mean_p(d(S.LOOP, S.FIRST_STEP)),
        "later_step_each": mean_p(later[multi] / (steps[multi] - 1)) if multi.any() else None,
        "tile_loop": mean_p(d(S.LOOP, S.LOOP_END)),
        "epilogue": mean_p(d(S.LOOP_END, S.END)),
        "item": mean_p(wg_end - wg_start),
        "tiles": mean_p(steps),
    }
    per_cu = collections.defaultdict(list)
    for i in np.argsort(wg_start):
        per_cu[int(cu[i])].append(int(i))
    pro, loop, epi, gaps, tail, head, count = [], [], [], [], [], [], []
    for idx in per_cu.values():
        pro.append(d(S.ENTRY, S.LOOP)[idx].sum())
        loop.append(d(S.LOOP, S.LOOP_END)[idx].sum())
        epi.append(d(S.LOOP_END, S.END)[idx].sum())
        gaps.append(sum(max(0.0, wg_start[b] - wg_end[a]) for a, b in zip(idx, idx[1:])))
        tail.append(base + span - wg_end[idx].max())
        head.append(wg_start[idx].min() - base)
        count.append(len(idx))
    cu_sum = {"prologue": float(np.mean(pro)), "tile_loop": float(np.mean(loop)), "epilogue": float(np.mean(epi)),
              "gaps": float(np.mean(gaps)), "head_idle": float(np.mean(head)), "tail_idle": float(np.mean(tail))}
    by_tiles = {}
    for lo, hi in ((1, 8), (9, 32), (33, 64), (65, 256), (257, 1 << 16)):
        m = (steps >= lo) & (steps <= hi) & multi
        if m.any():
            by_tiles[f"{lo}-{hi}"] = float(np.mean(later[m] / (steps[m] - 1)))
    per_xcd = {}
    for x in sorted(set(xcc.tolist())):
        m = xcc == x
        per_xcd[int(x)] = {"items": int(m.sum()), "last_end_us": float(wg_end[m].max() - base),
                           "later_step_us": float(np.mean(later[m & multi] / (steps[m & multi] - 1)))
                           if (m & multi).any() else None}
    return {"workgroups": int(r.shape[0]), "cus": len(per_cu), "workgroups_per_cu": float(np.mean(count)),
            "kernel_span_us": float(span), "per_item_us": item, "per_cu_us": cu_sum,
            "per_cu_share": {k: v / span for k, v in cu_sum.items()},
            "later_step_us_by_tiles": by_tiles, "per_xcd": per_xcd}


def summarize_roles(rec: np.ndarray, bins: int = 10) -> dict:
    """The fused mixed step: when the decode-role and prefill-role workgroups ran, and on how many CUs."""
    r = rec.astype(np.int64)
    r = r[(r[:, :, 6] > 0).all(axis=1)]
    dec = r[:, 0, 7] < 0
    start, end = r[:, :, 0].min(1) * TICK_US, r[:, :, 6].max(1) * TICK_US
    base = start.min()
    start, end = start - base, end - base
    span = end.max()
    cu = (((r[:, 0, 7] >> 16) & 0xF) << 8) | ((r[:, 0, 7] >> 8) & 0xFF)
    out = {"span_us": float(span)}
    for role, m in (("decode", dec), ("prefill", ~dec)):
        if not m.any():
            continue
        out[role] = {"workgroups": int(m.sum()), "cus": int(len(set(cu[m].tolist()))),
                     "first_start_us": float(start[m].min()), "last_end_us": float(end[m].max()),
                     "end_p10_us": float(np.percentile(end[m], 10)), "end_p50_us": float(np.percentile(end[m], 50)),
                     "end_p90_us": float(np.percentile(end[m], 90)),
                     "busy_cu_us": float((end[m] - start[m]).sum())}
    # CUs busy with each role, averaged over equal slices of the span
    edges = np.linspace(0.0, span, bins + 1)
    occ = {"decode": [], "prefill": []}
    for a, b in zip(edges, edges[1:]):
        for role, m in (("decode", dec), ("prefill", ~dec)):
            ov = np.clip(np.minimum(end[m], b) - np.maximum(start[m], a), 0.0, None)
            occ[role].append(float(ov.sum() / (b - a)))
    out["cus_busy_by_slice"] = occ
    out["slice_us"] = float(span / bins)
    return out


def markdown_roles(name: str, res: dict, cmd: str) -> str:
    lines = [f"# Phase stamps: the fused mixed-step kernel, {name}", "", f"Command: `{cmd}`.", "",
             f"Kernel span {res['span_us']:.1f} us (first workgroup start to last workgroup end, s_memrealtime at "
             "100 MHz).  The decode role is the first workgroups of the grid; each runs its wavefronts' share of "
             "the decode split, then every other workgroup runs one prefill work item.", "",
             "| role | workgroups | CUs | first start (us) | end p10 | end p50 | end p90 | last end | CU-us |",
             "|---|---|---|---|---|---|---|---|---|"]
    for role in ("decode", "prefill"):
        if role in res:
            v = res[role]
            lines.append(f"| {role} | {v['workgroups']} | {v['cus']} | {v['first_start_us']:.1f} | "
                         f"{v['end_p10_us']:.1f} | {v['end_p50_us']:.1f} | {v['end_p90_us']:.1f} | "
                         f"{v['last_end_us']:.1f} | {v['busy_cu_us']:.0f} |")
    lines += ["", f"CUs busy with each role, mean over slices of {res['slice_us']:.1f} us:", "",
              "| slice | " + " | ".join(str(i) for i in range(len(res["cus_busy_by_slice"]["decode"]))) + " |",
              "|---|" + "---|" * len(res["cus_busy_by_slice"]["decode"])]
    for role in ("decode", "prefill"):
        lines.append(f"| {role} | " + " | ".join(f"{x:.0f}" for x in res["cus_busy_by_slice"][role]) + " |")
    return "\n".join(lines) + "\n"


def markdown(name: str, res: dict, cmd: str) -> str:
    it, cu = res["per_item_us"], res["per_cu_us"]
    lines = [f"# Phase stamps: bf16 prefill attention, {name}", "",
             f"Command: `{cmd}`.", "",
             f"{res['workgroups']} work items on {res['cus']} CUs ({res['workgroups_per_cu']:.1f} per CU), "
             f"kernel span {res['kernel_span_us']:.1f} us (first wavefront start to last wavefront end, "
             "s_memrealtime at 100 MHz).", "",
             "Per work item (mean over the workgroup's wavefronts, then mean / p10 / p90 over items):", "",
             "| phase | mean (us) | p10 | p90 |", "|---|---|---|---|"]
    for k in ("issue_loads", "q_normalise_rotate", "tile0_to_loop", "prologue", "first_step", "later_step_each",
              "tile_loop", "epilogue", "item", "tiles"):
        v = it[k]
        if v is not None:
            label = "K/V tiles per item (count)" if k == "tiles" else k
            lines.append(f"| {label} | {v['mean']:.2f} | {v['p10']:.2f} | {v['p90']:.2f} |")
    lines += ["", "Per CU (sum over the items it ran, mean over CUs) and share of the kernel span:", "",
              "| part | us | share |", "|---|---|---|"]
    for k, v in cu.items():
        lines.append(f"| {k} | {v:.1f} | {100 * res['per_cu_share'][k]:.1f}% |")
    if res["later_step_us_by_tiles"]:
        lines += ["", "Later steps (after the first), us per step, by the item's tile count: " +
                  ", ".join(f"{k}: {v:.2f}" for k, v in res["later_step_us_by_tiles"].items()) + "."]
    if res.get("per_xcd"):
        lines += ["", "Per XCD (XCC_ID): items, last item end (us from the kernel's start), later-step time (us):", "",
                  "| XCD | " + " | ".join(str(x) for x in res["per_xcd"]) + " |",
                  "|---|" + "---|" * len(res["per_xcd"])]
        lines.append("| items | " + " | ".join(str(v["items"]) for v in res["per_xcd"].values()) + " |")
        lines.append("| last end | " + " | ".join(f"{v['last_end_us']:.0f}" for v in res["per_xcd"].values()) + " |")
        lines.append("| step | " + " | ".join("-" if v["later_step_us"] is None else f"{v['later_step_us']:.2f}"
                                                 for v in res["per_xcd"].values()) + " |")
    return "\n".join(lines) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="prefill_4x4096_qwen3_8b")
    ap.add_argument("--warmup-seconds", type=float, default=0.5)
    ap.add_argument("--no-weight-bound", action="store_true",
                    help="do not pass the norm weights' bound (both softmax kernels are launched)")
    ap.add_argument("--json", action="store_true", help="print the summary as one JSON line")
    ap.add_argument("--library", default=STAMPS_LIB_PATH,
                    help="a library built with -DQKRA_PHASE_STAMPS (default: the package's profiling build)")
    args = ap.parse_args(argv)
    import torch

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    from workloads import build_workload

    da = _load(os.path.abspath(args.library))
    w = build_workload(args.workload, device="cuda:0", parity=False)
    mixed = w.prefill is not None and w.decode is not None
    if mixed:
        call = _mixed_call(da, torch, w)
    else:
        call, _, _, _ = _prefill_call(da, torch, w, not args.no_weight_bound)
    torch.cuda.synchronize()
    t_end = time.perf_counter() + args.warmup_seconds
    while time.perf_counter() < t_end:
        for _ in range(5):
            call()
        torch.cuda.synchronize()
    da.check(da.qkra_phase_stamps_clear(), "qkra_phase_stamps_clear")
    call()
    torch.cuda.synchronize()
    nbytes = da.qkra_phase_stamps_bytes()
    host = np.zeros(nbytes // 8, dtype=np.uint64)
    da.check(da.qkra_phase_stamps_read(host, nbytes), "qkra_phase_stamps_read")
    rec = host.reshape(-1, 8, 8)
    res = summarize(rec)
    cmd = "python3 -m decoder_attention_amd.phase_stamps --workload " + args.workload
    if args.no_weight_bound:
        cmd += " --no-weight-bound"
    if mixed:
        roles = summarize_roles(rec)
        if args.json:
            print(json.dumps({"workload": args.workload, "roles": roles, "prefill_items": res}))
        else:
            print(markdown_roles(args.workload, roles, cmd), end="")
            print()
            print(markdown(args.workload + " (the prefill role's items)", res, cmd).split("\n", 4)[4], end="")
    elif args.json:
        print(json.dumps({"workload": args.workload, **res}))
    else:
        print(markdown(args.workload, res, cmd), end="")
    return 0


if __name__ == "__main__":
    sys.exit(main())
