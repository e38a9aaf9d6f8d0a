"""CPU fp64 oracle for QK-norm + RoPE + causal grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

It is the plain definition of the attention layer's forward pass, written out
in float64 NumPy, step by step in the order the pages give:

1. split the packed qkv row into Q, K and V heads;
2. RMS-normalise each Q and K head over its last dimension and scale by the
   learned weight (V untouched);
3. rotate Q and K with RoPE at the token's position;
4. store K and V in the per-request cache;
5. causal grouped-query softmax attention, scores scaled by 1/sqrt(D).

Three modes: ``prefill`` (packed requests, empty caches), ``decode`` (one new
token per request on a filled cache) and ``prefill_append`` (a chunk of new
tokens per request on a filled cache; it contains the other two).

Sources (page title, then section):
* zero-to-sglang, "Chapter 3 Forward Pass and Generation (Code Walkthrough)",
  section 3.3 "QKV, RoPE, and causal attention": the split, per-head Q/K
  RMSNorm, RoPE at token positions, KV-head repetition by whole groups, the
  1/sqrt(D) scale, the lower-triangular mask, float softmax and the product
  with V.  Section 3.1: packed ``[N, C]`` batches of several requests.
* zero-to-sglang, "Chapter 3 Forward Pass and Generation" (concept chapter),
  section 2.2 (RoPE rotates Q and K so dot products carry relative position),
  section 2.6 (RMSNorm drops mean centring; GQA shares K/V heads), section 4
  (prefill builds the K/V cache, decode adds one token that attends to the
  cached history).
* jq-wei, "transformer basics", "Attention calculation: part 1" (norm applied
  to the ``[..., H, D]`` view, ``scaling = head_dim ** -0.5``, output reshaped
  to ``[T, Hq*D]``) and "Prefill vs Decode" (the cache grows by one entry per
  decode step before attention runs).

Readings where the pages leave a detail open (each is listed, with its reason,
in the project's design notes):
* RoPE pairs element i with element i + D/2 ("rotate half"), with
  theta_i = base ** (-2 i / D); the pages fix neither the pairing nor the
  frequencies ("parity unpinned by the pages" for those two choices).
* RMSNorm puts eps inside the square root: x / sqrt(mean(x^2) + eps) * w.
* Decode writes the new token at slot L_b first and then attends over slots
  0..L_b, so a decode step equals the last row of a prefill over L_b+1 tokens.
* Requests never attend to each other; the causal index is the in-request one.
"""

from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step 1: split.  Columns [0, Hq*D) are Q heads, then Hkv K heads, then Hkv V
# heads, each D wide (code walkthrough 3.3; "transformer basics", part 1,
# [1,12,4096] -> [1,12,32,128] and [1,12,1024] -> [1,12,8,128]).
# ---------------------------------------------------------------------------

def split_qkv(qkv, num_q_heads: int, num_kv_heads: int, head_dim: int):
    qkv = _f64(qkv)
    n = qkv.shape[0]
    width = (num_q_heads + 2 * num_kv_heads) * head_dim
    if qkv.shape[1] != width:
        raise ValueError(f"qkv has {qkv.shape[1]} columns, expected {width}")
    q_end = num_q_heads * head_dim
    k_end = q_end + num_kv_heads * head_dim
    q = qkv[:, :q_end].reshape(n, num_q_heads, head_dim)
    k = qkv[:, q_end:k_end].reshape(n, num_kv_heads, head_dim)
    v = qkv[:, k_end:].reshape(n, num_kv_heads, head_dim)
    return q, k, v


# ---------------------------------------------------------------------------
# Step 2: RMSNorm over the last (head) dimension, weighted.
# ---------------------------------------------------------------------------

def rms_norm(x, weight, eps: float) -> np.ndarray:
    x = _f64(x)
    mean_square = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(mean_square + float(eps)) * _f64(weight)


# ---------------------------------------------------------------------------
# Step 3: RoPE, rotate-half pairing.  Pair (i, i + D/2) is turned by the
# angle p * theta_i with theta_i = base^(-2i/D).
# ---------------------------------------------------------------------------

def rope_frequencies(head_dim: int, base: float) -> np.ndarray:
    if head_dim % 2:
        raise ValueError("head_dim must be even for RoPE")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope_rotate_half(x, positions, base: float) -> np.ndarray:
    """x: [N, H, D]; positions: [N]."""
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    angle = _f64(positions)[:, None] * rope_frequencies(d, base)[None, :]   # [N, D/2]
    cos = np.cos(angle)[:, None, :]
    sin = np.sin(angle)[:, None, :]
    first, second = x[..., :half], x[..., half:]
    return np.concatenate([first * cos - second * sin, second * cos + first * sin], axis=-1)


def qk_norm_rope(qkv, q_norm_weight, k_norm_weight, positions, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, rms_eps: float, rope_base: float):
    """Steps 1-3 for a batch of rows: returns (q~ [N,Hq,D], k~ [N,Hkv,D], v [N,Hkv,D])."""
    q, k, v = split_qkv(qkv, num_q_heads, num_kv_heads, head_dim)
    q_t = rope_rotate_half(rms_norm(q, q_norm_weight, rms_eps), positions, rope_base)
    k_t = rope_rotate_half(rms_norm(k, k_norm_weight, rms_eps), positions, rope_base)
    return q_t, k_t, v


# ---------------------------------------------------------------------------
# Step 5: softmax attention of query rows against a prefix of keys.
# ---------------------------------------------------------------------------

def softmax(scores, axis: int = -1) -> np.ndarray:
    scores = _f64(scores)
    top = np.max(scores, axis=axis, keepdims=True)
    e = np.exp(scores - top)
    return e / np.sum(e, axis=axis, keepdims=True)


def causal_gqa_attention(q, k, v, return_probs: bool = False, block: int = 1024):
    """One request.  q: [T, Hq, D]; k, v: [T, Hkv, D]  ->  out [T, Hq, D].

    Query head h reads KV head floor(h / G) with G = Hq / Hkv (the pages
    repeat each KV head G times in a row).  Row i sees keys 0..i.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    t, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be divisible by Hkv")
    group = hq // hkv
    scale = 1.0 / np.sqrt(d)
    out = np.empty_like(q)
    probs = np.zeros((hq, t, t)) if return_probs else None
    for h in range(hq):
        g = h // group
        kt = k[:, g, :]
        vt = v[:, g, :]
        for r0 in range(0, t, block):
            r1 = min(t, r0 + block)
            s = (q[r0:r1, h, :] @ kt[:r1].T) * scale                   # [rows, r1]
            rows = np.arange(r0, r1)[:, None]
            cols = np.arange(r1)[None, :]
            s = np.where(cols <= rows, s, -np.inf)
            p = softmax(s, axis=-1)
            out[r0:r1, h, :] = p @ vt[:r1]
            if probs is not None:
                probs[h, r0:r1, :r1] = p
    if return_probs:
        return out, probs
    return out


def attend_prefix(q_row, keys, values) -> np.ndarray:
    """One query head row against keys/values [S, D] (all visible)."""
    q_row, keys, values = _f64(q_row), _f64(keys), _f64(values)
    s = (keys @ q_row) / np.sqrt(q_row.shape[-1])
    return softmax(s) @ values


# ---------------------------------------------------------------------------
# The two modes.
# ---------------------------------------------------------------------------

def prefill(qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, num_q_heads: int,
            num_kv_heads: int, head_dim: int, rms_eps: float, rope_base: float,
            cache_capacity: int, k_cache=None, v_cache=None) -> Dict[str, np.ndarray]:
    """Prefill of packed requests.

    Request r owns rows cu[r]..cu[r+1]-1; its token j goes to cache slot j.
    Returns ``out`` [N, Hq*D], ``q_tilde``, ``k_tilde``, ``v`` (per row) and
    the caches [B, Hkv, S_cap, D] (initial contents kept in untouched slots).
    """
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    b = len(cu) - 1
    q_t, k_t, v = qk_norm_rope(qkv, q_norm_weight, k_norm_weight, positions, num_q_heads,
                               num_kv_heads, head_dim, rms_eps, rope_base)
    n = q_t.shape[0]
    shape = (b, num_kv_heads, cache_capacity, head_dim)
    kc = np.full(shape, np.nan) if k_cache is None else _f64(k_cache).copy()
    vc = np.full(shape, np.nan) if v_cache is None else _f64(v_cache).copy()
    out = np.zeros((n, num_q_heads, head_dim))
    for r in range(b):
        lo, hi = cu[r], cu[r + 1]
        if hi - lo > cache_capacity:
            raise ValueError("request longer than the cache capacity")
        if hi == lo:
            continue
        kc[r, :, : hi - lo, :] = np.transpose(k_t[lo:hi], (1, 0, 2))
        vc[r, :, : hi - lo, :] = np.transpose(v[lo:hi], (1, 0, 2))
        out[lo:hi] = causal_gqa_attention(q_t[lo:hi], k_t[lo:hi], v[lo:hi])
    return {"out": out.reshape(n, num_q_heads * head_dim), "q_tilde": q_t, "k_tilde": k_t,
            "v": v, "k_cache": kc, "v_cache": vc}


def prefill_rows(q_tilde, k_tilde, v, cu_seqlens, tokens: Iterable[int]) -> Dict[int, np.ndarray]:
    """Output rows [Hq, D] for selected packed token indices, from keys 0..i alone.

    Used at sizes where the full prefill is too slow: row i of a request
    depends on its keys 0..i only, so any sample of rows can be checked.
    """
    q_tilde, k_tilde, v = _f64(q_tilde), _f64(k_tilde), _f64(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    hq, d = q_tilde.shape[1], q_tilde.shape[2]
    hkv = k_tilde.shape[1]
    group = hq // hkv
    result = {}
    for n in tokens:
        n = int(n)
        r = int(np.searchsorted(cu, n, side="right") - 1)
        lo = int(cu[r])
        rows = np.empty((hq, d))
        for g in range(hkv):
            keys = k_tilde[lo:n + 1, g, :]
            vals = v[lo:n + 1, g, :]
            q = q_tilde[n, g * group:(g + 1) * group, :]               # [G, D]
            s = (q @ keys.T) / np.sqrt(d)
            rows[g * group:(g + 1) * group] = softmax(s, axis=-1) @ vals
        result[n] = rows
    return result


def decode(qkv, q_norm_weight, k_norm_weight, positions, cache_lens, k_cache, v_cache,
           num_q_heads: int, num_kv_heads: int, head_dim: int, rms_eps: float,
           rope_base: float) -> Dict[str, np.ndarray]:
    """One new token per request.

    The new token's K~ and V go to slot L_b of request b's cache, then its
    query attends over slots 0..L_b (the cached history plus itself).
    ``k_cache``/``v_cache``: [B, Hkv, S, D] with at least L_b + 1 slots.
    """
    q_t, k_t, v = qk_norm_rope(qkv, q_norm_weight, k_norm_weight, positions, num_q_heads,
                               num_kv_heads, head_dim, rms_eps, rope_base)
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache).copy()
    lens = [int(x) for x in np.asarray(cache_lens).tolist()]
    b = len(lens)
    group = num_q_heads // num_kv_heads
    out = np.zeros((b, num_q_heads, head_dim))
    for i in range(b):
        L = lens[i]
        if L + 1 > kc.shape[2]:
            raise ValueError("cache capacity too small for the new token")
        kc[i, :, L, :] = k_t[i]
        vc[i, :, L, :] = v[i]
        for h in range(num_q_heads):
            g = h // group
            out[i, h] = attend_prefix(q_t[i, h], kc[i, g, : L + 1], vc[i, g, : L + 1])
    return {"out": out.reshape(b, num_q_heads * head_dim), "q_tilde": q_t, "k_tilde": k_t,
            "v": v, "k_cache": kc, "v_cache": vc}


def prefill_append(qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, cache_lens, k_cache, v_cache,
                   num_q_heads: int, num_kv_heads: int, head_dim: int, rms_eps: float,
                   rope_base: float, block: int = 1024) -> Dict[str, np.ndarray]:
    """A chunk of new tokens per request, appended to a cache that already holds entries.

    Request r owns packed rows cu[r]..cu[r+1]-1, its T_r new tokens, on top of
    P_r = cache_lens[r] cached entries.  New token j goes to slot P_r + j and
    its query attends over slots 0..P_r + j: the cached history, the chunk's
    earlier tokens and itself (concept chapter, section 4: prefill builds the
    cache and later tokens attend to the cached history; "Prefill vs Decode":
    the cache grows before attention runs).  P_r = 0 is a prefill, T_r = 1 a
    decode step.  ``k_cache``/``v_cache``: [B, Hkv, S, D] with S >= P_r + T_r.
    """
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    lens = [int(x) for x in np.asarray(cache_lens).tolist()]
    q_t, k_t, v = qk_norm_rope(qkv, q_norm_weight, k_norm_weight, positions, num_q_heads,
                               num_kv_heads, head_dim, rms_eps, rope_base)
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache).copy()
    n = q_t.shape[0]
    group = num_q_heads // num_kv_heads
    scale = 1.0 / np.sqrt(head_dim)
    out = np.zeros((n, num_q_heads, head_dim))
    for r in range(len(lens)):
        lo, hi, past = cu[r], cu[r + 1], lens[r]
        t = hi - lo
        if past + t > kc.shape[2]:
            raise ValueError("cache capacity too small for the appended chunk")
        if t == 0:
            continue
        kc[r, :, past:past + t, :] = np.transpose(k_t[lo:hi], (1, 0, 2))
        vc[r, :, past:past + t, :] = np.transpose(v[lo:hi], (1, 0, 2))
        for h in range(num_q_heads):
            g = h // group
            keys, values = kc[r, g, : past + t], vc[r, g, : past + t]
            for r0 in range(0, t, block):
                r1 = min(t, r0 + block)
                s = (q_t[lo + r0:lo + r1, h, :] @ keys.T) * scale               # [rows, past + t]
                rows = past + np.arange(r0, r1)[:, None]                       # slot of each query
                cols = np.arange(past + t)[None, :]
                p = softmax(np.where(cols <= rows, s, -np.inf), axis=-1)
                out[lo + r0:lo + r1, h, :] = p @ values
    return {"out": out.reshape(n, num_q_heads * head_dim), "q_tilde": q_t, "k_tilde": k_t,
            "v": v, "k_cache": kc, "v_cache": vc}


# ---------------------------------------------------------------------------
# Diagnostics: bfloat16 storage rounding (round to nearest, ties to even), to
# separate the error of storing K~ in a bf16 cache from the kernels' own.
# ---------------------------------------------------------------------------

def round_to_bf16(x) -> np.ndarray:
    f = np.ascontiguousarray(_f64(x).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)
