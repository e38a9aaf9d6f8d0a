"""CPU fp64 oracle for the attention layer over a paged K/V cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

The pages introduce the per-request K/V cache (prefill fills it, each decode
step appends one entry: zero-to-sglang "Chapter 3 Forward Pass and Generation",
section 4; jq-wei "transformer basics", "Prefill vs Decode") and defer its
optimised, paged form to a later chapter that they only name ("Chapter 4: KV
Cache Optimization" in the code walkthrough's opening and references).  The
reading taken here is the plainest one that leaves every result unchanged: a
paged cache is the same per-request cache with its slots stored in fixed-size
pages of a shared pool, found through a block table.

* Pool: ``k_pool``, ``v_pool`` of shape [num_pages, Hkv, P, D]; a page holds P
  consecutive slots of one request for every KV head.
* Block table: int [B, pages_per_seq]; slot s of request b is row s % P of
  page ``table[b][s // P]``.
* Everything the attention computes is defined on the logical cache those
  slots form, exactly as for the contiguous cache (``qknorm_rope_attn``).

So the oracle gathers each request's logical cache from the pool, runs the
contiguous definition on it, and writes the slots the call adds back through
the same table.  Pages that no written slot maps to keep their contents.
"""

from __future__ import annotations

from typing import Dict, Sequence

import numpy as np

from . import qknorm_rope_attn as contiguous


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def page_of(table, b: int, s: int, page_size: int):
    """(page, row) holding slot s of request b."""
    return int(np.asarray(table)[b, s // page_size]), s % page_size


def gather(pool, table, request: int, num_slots: int, page_size: int) -> np.ndarray:
    """Request `request`'s logical cache [Hkv, num_slots, D] from the pool."""
    pool = _f64(pool)
    hkv, d = pool.shape[1], pool.shape[3]
    out = np.empty((hkv, num_slots, d))
    for s in range(num_slots):
        page, row = page_of(table, request, s, page_size)
        out[:, s, :] = pool[page, :, row, :]
    return out


def scatter(pool: np.ndarray, table, request: int, slots: Sequence[int], values, page_size: int) -> None:
    """Writes values[:, i, :] (shape [Hkv, len(slots), D]) to slot slots[i] of `request`, in place."""
    values = _f64(values)
    for i, s in enumerate(slots):
        page, row = page_of(table, request, int(s), page_size)
        pool[page, :, row, :] = values[:, i, :]


def decode(qkv, q_norm_weight, k_norm_weight, positions, cache_lens, k_pool, v_pool, block_table,
           page_size: int, num_q_heads: int, num_kv_heads: int, head_dim: int, rms_eps: float,
           rope_base: float) -> Dict[str, np.ndarray]:
    """One new token per request on a paged cache: slot L_b is written through the table, then the query
    attends over slots 0..L_b (the contiguous decode on the request's logical cache)."""
    lens = [int(x) for x in np.asarray(cache_lens).tolist()]
    kp, vp = _f64(k_pool).copy(), _f64(v_pool).copy()
    qkv = _f64(qkv)
    outs, kts = [], []
    for b, L in enumerate(lens):
        kc = gather(kp, block_table, b, L + 1, page_size)[None]     # slot L: whatever the pool holds there
        vc = gather(vp, block_table, b, L + 1, page_size)[None]
        res = contiguous.decode(qkv[b:b + 1], q_norm_weight, k_norm_weight, np.asarray(positions)[b:b + 1], [L],
                                kc, vc, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                                rms_eps=rms_eps, rope_base=rope_base)
        scatter(kp, block_table, b, [L], res["k_cache"][0][:, L:L + 1, :], page_size)
        scatter(vp, block_table, b, [L], res["v_cache"][0][:, L:L + 1, :], page_size)
        outs.append(res["out"][0])
        kts.append(res["k_tilde"][0])
    width = num_q_heads * head_dim
    return {"out": np.array(outs).reshape(len(lens), width), "k_tilde": np.array(kts).reshape(len(lens),
                                                                                            num_kv_heads, head_dim),
            "k_pool": kp, "v_pool": vp}


def prefill_append(qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, cache_lens, k_pool, v_pool,
                   block_table, page_size: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   rms_eps: float, rope_base: float) -> Dict[str, np.ndarray]:
    """A chunk of T_r new tokens per request on a paged cache holding P_r entries (P_r = 0: a prefill): token j
    goes to slot P_r + j through the table and attends over slots 0..P_r + j."""
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    lens = [int(x) for x in np.asarray(cache_lens).tolist()]
    kp, vp = _f64(k_pool).copy(), _f64(v_pool).copy()
    qkv = _f64(qkv)
    pos = np.asarray(positions)
    n = qkv.shape[0]
    out = np.zeros((n, num_q_heads * head_dim))
    k_tilde = np.zeros((n, num_kv_heads, head_dim))
    for r, past in enumerate(lens):
        lo, hi = cu[r], cu[r + 1]
        t = hi - lo
        if t == 0:
            continue
        kc = gather(kp, block_table, r, past + t, page_size)[None]
        vc = gather(vp, block_table, r, past + t, page_size)[None]
        res = contiguous.prefill_append(qkv[lo:hi], q_norm_weight, k_norm_weight, pos[lo:hi], [0, t], [past], kc,
                                        vc, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                                        head_dim=head_dim, rms_eps=rms_eps, rope_base=rope_base)
        slots = list(range(past, past + t))
        scatter(kp, block_table, r, slots, res["k_cache"][0][:, past:past + t, :], page_size)
        scatter(vp, block_table, r, slots, res["v_cache"][0][:, past:past + t, :], page_size)
        out[lo:hi] = res["out"]
        k_tilde[lo:hi] = res["k_tilde"]
    return {"out": out, "k_tilde": k_tilde, "k_pool": kp, "v_pool": vp}
