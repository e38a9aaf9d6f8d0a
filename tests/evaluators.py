"""Independent CPU evaluators used to pin the oracle (they share no code with it).

* ``grouped_attention`` -- the attention step stated as its definition
  (zero-to-sglang code walkthrough, section 3.3): row i of query head h takes
  softmax over the visible keys j <= i of q_i . k_j / sqrt(D), with k and v
  from KV head h // G, and sums the visible values with those weights.  The KV
  heads are indexed by group (one contraction per group of query heads) and
  the visible set is built from the indices; torch float64 on the CPU.
* ``library_attention`` -- torch's own ``scaled_dot_product_attention`` with
  ``is_causal=True`` (a library routine), float64 on the CPU.
* ``brute_force_layer`` -- the whole layer (split, RMSNorm, RoPE, causal GQA
  attention) as scalar Python loops with the ``math`` module, for tiny inputs.
"""

from __future__ import annotations

import math
from typing import List, Sequence

import torch


def grouped_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    """q: [1, Hq, T, D]; k, v: [1, Hkv, T, D] (float64).  Returns (out [1, Hq, T, D], probs [1, Hq, T, T])."""
    hq, t, d = q.shape[1], q.shape[2], q.shape[3]
    hkv = k.shape[1]
    group = hq // hkv
    # Query head h = g * group + c belongs to KV head g: view the heads as [g, c].
    qg = q[0].reshape(hkv, group, t, d)
    logits = torch.einsum("gcid,gjd->gcij", qg, k[0]) / math.sqrt(d)        # [Hkv, G, query i, key j]
    visible = torch.arange(t)[None, :] <= torch.arange(t)[:, None]          # [i, j]: key j at or before row i
    top = torch.where(visible, logits, torch.full_like(logits, -math.inf)).amax(dim=-1, keepdim=True)
    weight = torch.where(visible, torch.exp(logits - top), torch.zeros_like(logits))
    probs = weight / weight.sum(dim=-1, keepdim=True)
    out = torch.einsum("gcij,gjd->gcid", probs, v[0])
    return out.reshape(1, hq, t, d), probs.reshape(1, hq, t, t)


def library_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, native_gqa: bool = False):
    """torch SDPA, causal.  Layouts as in ``grouped_attention``."""
    f = torch.nn.functional.scaled_dot_product_attention
    if native_gqa:
        return f(q, k, v, is_causal=True, enable_gqa=True)
    group = q.shape[1] // k.shape[1]
    return f(q, k.repeat_interleave(group, dim=1), v.repeat_interleave(group, dim=1), is_causal=True)


def brute_force_layer(qkv: Sequence[Sequence[float]], q_weight: Sequence[float],
                      k_weight: Sequence[float], positions: Sequence[int], seqlens: Sequence[int],
                      hq: int, hkv: int, d: int, eps: float, base: float) -> List[List[List[float]]]:
    """Scalar loops over the whole layer; returns out[n][h][dim]."""
    half = d // 2

    def head(row, col0):
        return [float(row[col0 + i]) for i in range(d)]

    def norm(x, w):
        ms = sum(e * e for e in x) / d
        r = 1.0 / math.sqrt(ms + eps)
        return [x[i] * r * float(w[i]) for i in range(d)]

    def rotate(x, p):
        y = [0.0] * d
        for i in range(half):
            a = p * base ** (-(2.0 * i) / d)
            c, s = math.cos(a), math.sin(a)
            y[i] = x[i] * c - x[i + half] * s
            y[i + half] = x[i + half] * c + x[i] * s
        return y

    qs, ks, vs = [], [], []
    for n, row in enumerate(qkv):
        p = positions[n]
        qs.append([rotate(norm(head(row, h * d), q_weight), p) for h in range(hq)])
        ks.append([rotate(norm(head(row, (hq + g) * d), k_weight), p) for g in range(hkv)])
        vs.append([head(row, (hq + hkv + g) * d) for g in range(hkv)])

    group = hq // hkv
    out = []
    start = 0
    for t in seqlens:
        for i in range(t):
            n = start + i
            rows = []
            for h in range(hq):
                g = h // group
                scores = []
                for j in range(i + 1):
                    dot = sum(qs[n][h][e] * ks[start + j][g][e] for e in range(d))
                    scores.append(dot / math.sqrt(d))
                top = max(scores)
                w = [math.exp(s - top) for s in scores]
                z = sum(w)
                rows.append([sum(w[j] * vs[start + j][g][e] for j in range(i + 1)) / z
                             for e in range(d)])
            out.append(rows)
        start += t
    return out
