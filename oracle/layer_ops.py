"""CPU fp64 oracle for the decoder-layer steps around attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

Two steps the pages place next to the attention layer:

* The fused residual add + RMSNorm that sits before every attention and MLP
  sublayer (zero-to-sglang, "Chapter 3 Forward Pass and Generation (Code
  Walkthrough)", section 3.2 "Computation inside a decoder layer").  The first
  call of a model forward has no residual: it keeps x itself as the residual
  and returns RMSNorm(x).  Every later call first adds the sublayer output x to
  the residual stream, keeps the sum as the new residual and returns its
  RMSNorm.  Expanded, a layer is h = x + Attn(RMSNorm(x)) followed by
  out = h + MLP(RMSNorm(h)); the MLP's addition is deferred to the next
  layer's first norm, or to the model's final norm.
* Choosing the next token (same page, section 4.1 "Keep the last position of
  each request" and section 4.3 "Find sampling in the engine"): the LM head
  reads only each request's last packed row, and a fully greedy batch takes
  the argmax of every logits row.

Readings where the pages leave a detail open:
* RMSNorm is x / sqrt(mean(x^2) + eps) * w over the hidden dimension (the
  same form as the per-head Q/K norm).
* A request with no tokens has no last position: it selects no row.
* Argmax ties go to the lowest index (the pages fix no tie-break; this is the
  first-occurrence rule of the library argmax the page calls).  A NaN counts
  as larger than every number, so the first NaN of a row wins.
"""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .qknorm_rope_attn import rms_norm


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def fused_add_rms_norm(x, residual: Optional[np.ndarray], weight, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """One call of the fused residual add + RMSNorm (Code Walkthrough, section 3.2).

    ``x``: [N, C] sublayer output (or the embeddings on the first call);
    ``residual``: [N, C] residual stream, or None on the first call;
    ``weight``: [C].  Returns ``(normalised, new_residual)``: without a
    residual, new_residual = x; with one, new_residual = x + residual; the
    normalised output is RMSNorm(new_residual) * weight in both cases.
    """
    x = _f64(x)
    r = x.copy() if residual is None else x + _f64(residual)
    return rms_norm(r, weight, eps), r


def last_positions(cu_seqlens: Sequence[int]) -> np.ndarray:
    """Packed row index of each request's last token (Code Walkthrough, section 4.1).

    Request r owns rows cu[r] .. cu[r+1]-1; its last position is cu[r+1]-1.
    A request with no tokens gets -1 (it selects no row).
    """
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    return np.array([cu[r + 1] - 1 if cu[r + 1] > cu[r] else -1 for r in range(len(cu) - 1)], dtype=np.int64)


def gather_last(hidden, cu_seqlens: Sequence[int]) -> np.ndarray:
    """The rows ``hidden[last_positions(cu)]`` ([B, C]); rows of empty requests are NaN."""
    h = _f64(hidden)
    idx = last_positions(cu_seqlens)
    out = np.full((len(idx), h.shape[1]), np.nan)
    for r, i in enumerate(idx):
        if i >= 0:
            out[r] = h[i]
    return out


def greedy_argmax(logits) -> np.ndarray:
    """Per row, the index of the largest logit (Code Walkthrough, section 4.3).

    Ties go to the lowest index; a NaN counts as larger than every number.
    Written as a plain scan over each row.
    """
    z = _f64(logits)
    out = np.empty(z.shape[0], dtype=np.int64)
    for b in range(z.shape[0]):
        best = 0
        for j in range(1, z.shape[1]):
            if np.isnan(z[b, best]):
                break
            if np.isnan(z[b, j]) or z[b, j] > z[b, best]:
                best = j
        out[b] = best
    return out
