"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, compare."""

from __future__ import annotations

import sys
from typing import Dict, Iterable, Optional

import numpy as np
import torch

import decoder_attention_amd as da
import oracle

BF16_TOL = 2e-2   # max-abs error bound for bf16 inputs/outputs (fp32 accumulation)
FP32_TOL = 1e-4   # max-abs error bound in fp32 mode


def tol_for(dtype) -> float:
    return BF16_TOL if dtype == torch.bfloat16 else FP32_TOL


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def cfg_of(heads, dtype) -> da.QkraConfig:
    return da.make_config(heads.num_q_heads, heads.num_kv_heads, heads.head_dim, dtype, heads.rms_eps,
                          heads.rope_base)


def layer_kw(heads) -> dict:
    return dict(num_q_heads=heads.num_q_heads, num_kv_heads=heads.num_kv_heads, head_dim=heads.head_dim,
                rms_eps=heads.rms_eps, rope_base=heads.rope_base)


def run_prefill(p) -> Dict[str, torch.Tensor]:
    """HIP prefill on PrefillInputs (device tensors); caches are updated in place.  `out` starts as NaN, so a
    row that no kernel wrote fails any comparison."""
    cfg = cfg_of(p.heads, p.qkv.dtype)
    h = p.heads
    out = torch.full((p.num_tokens, h.num_q_heads * h.head_dim), float("nan"), dtype=p.qkv.dtype,
                     device=p.qkv.device)
    out, ws = da.prefill(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens,
                         p.max_seqlen, p.k_cache, p.v_cache, out=out)
    torch.cuda.synchronize()
    n, h = p.num_tokens, p.heads
    if p.qkv.dtype != torch.float32:  # bf16: Q is normalised and rotated inside the attention kernel
        return {"out": out, "q_tilde": None}
    q_tilde = ws[: n * h.num_q_heads * h.head_dim * p.qkv.element_size()].view(p.qkv.dtype)
    return {"out": out, "q_tilde": q_tilde.view(n, h.num_q_heads, h.head_dim)}


def run_decode(d, k_cache=None, v_cache=None) -> Dict[str, torch.Tensor]:
    cfg = cfg_of(d.heads, d.qkv.dtype)
    kc = d.k_cache if k_cache is None else k_cache
    vc = d.v_cache if v_cache is None else v_cache
    out, ws = da.decode(cfg, d.qkv, d.q_norm_weight, d.k_norm_weight, d.positions, d.cache_lens,
                        d.max_cache_len, kc, vc)
    torch.cuda.synchronize()
    return {"out": out}


def oracle_prefill(p, init_k=None, init_v=None):
    return oracle.prefill(f64(p.qkv), f64(p.q_norm_weight), f64(p.k_norm_weight), p.positions.cpu().numpy(),
                          p.cu_seqlens.cpu().numpy(), cache_capacity=p.cache_capacity,
                          k_cache=init_k, v_cache=init_v, **layer_kw(p.heads))


def oracle_decode_rows(qkv, q_norm_weight, k_norm_weight, positions, cache_lens, k_cache, v_cache, heads,
                       requests=None, chunk: int = 4) -> Dict[str, np.ndarray]:
    """oracle.decode for the listed requests (all if None), a few at a time.

    Each chunk's caches are cut to its longest history plus the new slot and widened to fp64 on their own, so a
    full-size decode (128 requests of up to 16k entries) fits in host memory.  The oracle still sees every cached
    entry of every request it checks.  Returns ``out`` [R, Hq*D] and ``k_tilde`` [R, Hkv, D] in request order.
    """
    lens = [int(x) for x in cache_lens.cpu().tolist()]
    pos = positions.cpu().numpy()
    requests = list(range(len(lens))) if requests is None else [int(b) for b in requests]
    outs, kts = [], []
    for c0 in range(0, len(requests), chunk):
        sub = requests[c0:c0 + chunk]
        top = max(lens[b] for b in sub) + 1
        idx = torch.tensor(sub, device=k_cache.device)
        ref = oracle.decode(f64(qkv.index_select(0, idx)), f64(q_norm_weight), f64(k_norm_weight), pos[sub],
                            np.array([lens[b] for b in sub]), f64(k_cache.index_select(0, idx)[:, :, :top]),
                            f64(v_cache.index_select(0, idx)[:, :, :top]), **layer_kw(heads))
        outs.append(ref["out"])
        kts.append(ref["k_tilde"])
    return {"out": np.concatenate(outs), "k_tilde": np.concatenate(kts)}


def check_decode_result(d, out: torch.Tensor, k_before: torch.Tensor, v_before: torch.Tensor, tol: float,
                        what: str = "decode", requests=None, k_rel: float = 0.0) -> float:
    """A decode's `out` and caches against the oracle: every listed request's output row (all if None), its new
    K slot within `tol` and its new V slot bit for bit; every slot other than L_b, of every request, unchanged."""
    h = d.heads
    hq, hkv, dim = h.num_q_heads, h.num_kv_heads, h.head_dim
    b_all = d.qkv.shape[0]
    requests = list(range(b_all)) if requests is None else list(requests)
    ref = oracle_decode_rows(d.qkv, d.q_norm_weight, d.k_norm_weight, d.positions, d.cache_lens, k_before,
                             v_before, h, requests)
    idx = torch.tensor(requests, device=out.device)
    err = assert_close(f64(out.index_select(0, idx)), ref["out"], tol, f"{what} out")
    lens = d.cache_lens.cpu().tolist()
    v_new = d.qkv[:, (hq + hkv) * dim:].reshape(b_all, hkv, dim)
    kb, vb = bits(d.k_cache), bits(d.v_cache)
    kb0, vb0 = bits(k_before), bits(v_before)
    rows = torch.arange(b_all, device=d.k_cache.device)
    lens_dev = d.cache_lens.long()
    assert torch.equal(vb[rows, :, lens_dev], bits(v_new)), f"{what}: a new V slot differs from the input V"
    new_k = f64(d.k_cache[rows, :, lens_dev])
    assert_close_k(new_k[requests], ref["k_tilde"], tol, k_rel, f"{what} new K slots")
    mask = torch.ones(d.k_cache.shape[:3], dtype=torch.bool, device=d.k_cache.device)
    mask[rows, :, lens_dev] = False
    assert torch.equal(kb[mask], kb0[mask]) and torch.equal(vb[mask], vb0[mask]), f"{what}: a slot other than L_b changed"
    assert len(lens) == b_all
    return err


def max_abs(got: np.ndarray, want: np.ndarray) -> float:
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - want)))


def assert_close(got: np.ndarray, want: np.ndarray, tol: float, what: str) -> float:
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in the HIP result"
    err = max_abs(got, want)
    if err > tol:
        idx = np.unravel_index(np.argmax(np.abs(got - want)), got.shape)
        raise AssertionError(f"{what}: max-abs error {err:.3e} > {tol:.1e} at {idx}: "
                             f"got {got[idx]!r} want {want[idx]!r}")
    return err


def bits(t: torch.Tensor) -> torch.Tensor:
    """Raw bit patterns of a tensor (exact comparisons, NaN payloads included)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    raise TypeError(t.dtype)


def assert_close_k(got: np.ndarray, want: np.ndarray, tol: float, k_rel: float, what: str) -> None:
    """K~ within tol + k_rel * |want|: with k_rel = 2^-8 this allows the half bf16 step of values past 8, where a
    correctly rounded bf16 alone is off by more than 2e-2 (large norm weights)."""
    if k_rel == 0.0:
        assert_close(got, want, tol, what)
        return
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.abs(got - want) > tol + k_rel * np.abs(want)
    assert not np.any(bad) and np.all(np.isfinite(got)), f"{what}: {int(bad.sum())} values outside tol + rel*|want|"


def check_prefill_caches(p, k_before: torch.Tensor, v_before: torch.Tensor, ref: dict, tol: float,
                         k_rel: float = 0.0) -> None:
    """V cache equals the input V bits; K cache matches the oracle's k~; untouched slots keep their bits."""
    h = p.heads
    hq, hkv, d = h.num_q_heads, h.num_kv_heads, h.head_dim
    cu = p.cu_seqlens.cpu().tolist()
    v_in = p.qkv[:, (hq + hkv) * d:].reshape(-1, hkv, d)
    kb, vb = bits(p.k_cache), bits(p.v_cache)
    kb0, vb0 = bits(k_before), bits(v_before)
    for r in range(p.num_seqs):
        lo, hi = cu[r], cu[r + 1]
        t = hi - lo
        if t:
            assert torch.equal(vb[r, :, :t], bits(v_in[lo:hi].permute(1, 0, 2).contiguous())), f"V cache request {r}"
            got = f64(p.k_cache[r, :, :t])
            assert_close_k(got, np.transpose(ref["k_tilde"][lo:hi], (1, 0, 2)), tol, k_rel, f"K cache request {r}")
        assert torch.equal(kb[r, :, t:], kb0[r, :, t:]), f"K cache slots >= {t} of request {r} were written"
        assert torch.equal(vb[r, :, t:], vb0[r, :, t:]), f"V cache slots >= {t} of request {r} were written"


def sample_tokens(cu: Iterable[int], per_request: int, seed: int, tile: int = 64) -> list:
    """Rows 0, 1, the last, tile edges and random ones of every request."""
    rng = np.random.default_rng(seed)
    cu = list(cu)
    rows = set()
    for r in range(len(cu) - 1):
        lo, hi = cu[r], cu[r + 1]
        t = hi - lo
        if t == 0:
            continue
        for i in (0, 1, t - 1, t - 2):
            if 0 <= i < t:
                rows.add(lo + i)
        for e in range(tile, t, tile * max(1, t // (tile * 8))):
            rows.update(x for x in (lo + e - 1, lo + e) if lo <= x < hi)
        rows.update(int(lo + x) for x in rng.integers(0, t, size=per_request))
    return sorted(rows)
