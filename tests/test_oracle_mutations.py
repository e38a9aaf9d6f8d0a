"""Each plausible mistake planted in a copy of an oracle function fails some pin.

The mistakes are planted on the CPU, in the oracle's module namespace, for the
duration of one test (pytest's monkeypatch restores the real functions).
"""

import math

import numpy as np
import pytest

import oracle.layer_ops as lo
import oracle.qknorm_rope_attn as orc
import pins

REAL = {name: getattr(orc, name) for name in
        ("split_qkv", "rms_norm", "rope_rotate_half", "rope_frequencies", "causal_gqa_attention",
         "attend_prefix", "qk_norm_rope", "softmax", "prefill_append")}


def _rope_sign(x, positions, base):
    y = REAL["rope_rotate_half"](x, positions, base)
    half = y.shape[-1] // 2
    z = REAL["rope_rotate_half"](x, -np.asarray(positions, dtype=np.float64), base)
    return np.concatenate([y[..., :half], z[..., half:]], axis=-1)


def _freq_exponent(head_dim, base):
    return np.power(float(base), -np.arange(head_dim // 2, dtype=np.float64) / head_dim)


def _eps_outside(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * np.asarray(w, dtype=np.float64)


def _no_weight(x, w, eps):
    return REAL["rms_norm"](x, np.ones_like(np.asarray(w, dtype=np.float64)), eps)


def _mean_not_rms(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    c = x - x.mean(axis=-1, keepdims=True)
    return REAL["rms_norm"](c, w, eps)


def _scale_one_over_d(q, k, v, return_probs=False, block=1024):
    q = np.asarray(q, dtype=np.float64)
    return REAL["causal_gqa_attention"](q / math.sqrt(q.shape[-1]), k, v, return_probs, block)


def _gqa_modulo(q, k, v, return_probs=False, block=1024):
    hq, hkv = np.shape(q)[1], np.shape(k)[1]
    idx = [h % hkv for h in range(hq)]
    return REAL["causal_gqa_attention"](q, np.asarray(k)[:, idx], np.asarray(v)[:, idx], return_probs, block)


def _mask_sees_next(q, k, v, return_probs=False, block=1024):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    t, hq, d = q.shape
    group = hq // k.shape[1]
    out = np.empty_like(q)
    probs = np.zeros((hq, t, t))
    for h in range(hq):
        s = q[:, h] @ k[:, h // group].T / math.sqrt(d)
        allowed = np.arange(t)[None, :] <= np.arange(t)[:, None] + 1
        s = np.where(allowed, s, -np.inf)
        p = REAL["softmax"](s)
        out[:, h] = p @ v[:, h // group]
        probs[h] = p
    return (out, probs) if return_probs else out


def _kv_swapped(qkv, hq, hkv, d):
    q, k, v = REAL["split_qkv"](qkv, hq, hkv, d)
    return q, v, k


def _v_normalised(qkv, wq, wk, positions, hq, hkv, d, eps, base):
    q, k, v = REAL["qk_norm_rope"](qkv, wq, wk, positions, hq, hkv, d, eps, base)
    return q, k, REAL["rms_norm"](v, np.ones(d), eps)


def _decode_without_self(q_row, keys, values):
    if len(keys) > 1:
        return REAL["attend_prefix"](q_row, keys[:-1], values[:-1])
    return REAL["attend_prefix"](q_row, keys, values)


def _softmax_no_norm(scores, axis=-1):
    s = np.asarray(scores, dtype=np.float64)
    return np.exp(s - np.max(s, axis=axis, keepdims=True))


def _append_ignores_history(qkv, wq, wk, positions, cu, cache_lens, k_cache, v_cache, *args, **kw):
    # The chunk attends only to itself: the cached entries are written over by a prefill.
    hist = np.asarray(cache_lens)
    res = REAL["prefill_append"](qkv, wq, wk, positions, cu, np.zeros_like(hist), k_cache, v_cache, *args, **kw)
    return res


def _append_writes_from_slot_zero(qkv, wq, wk, positions, cu, cache_lens, k_cache, v_cache, *args, **kw):
    res = REAL["prefill_append"](qkv, wq, wk, positions, cu, cache_lens, k_cache, v_cache, *args, **kw)
    lens = np.asarray(cache_lens)
    cu = np.asarray(cu)
    for r, past in enumerate(lens):
        t = int(cu[r + 1] - cu[r])
        if past > 0 and t > 0:  # the chunk's K lands at slot 0 instead of slot P_r
            res["k_cache"][r, :, :t] = res["k_cache"][r, :, past:past + t]
    return res


def _append_mask_excludes_self(qkv, wq, wk, positions, cu, cache_lens, k_cache, v_cache, num_q_heads,
                               num_kv_heads, head_dim, rms_eps, rope_base, block=1024):
    res = REAL["prefill_append"](qkv, wq, wk, positions, cu, cache_lens, k_cache, v_cache, num_q_heads,
                                 num_kv_heads, head_dim, rms_eps, rope_base, block)
    q_t, kc, vc = res["q_tilde"], res["k_cache"], res["v_cache"]
    out = res["out"].reshape(q_t.shape).copy()
    group = num_q_heads // num_kv_heads
    cu = np.asarray(cu)
    for r, past in enumerate(np.asarray(cache_lens)):
        for j in range(int(cu[r + 1] - cu[r])):
            n = int(cu[r]) + j
            if past + j == 0:
                continue
            for h in range(num_q_heads):
                g = h // group
                out[n, h] = REAL["attend_prefix"](q_t[n, h], kc[r, g, : past + j], vc[r, g, : past + j])
    res["out"] = out.reshape(res["out"].shape)
    return res


MUTANTS = {
    "append_ignores_history": ("prefill_append", _append_ignores_history),
    "append_writes_from_slot_zero": ("prefill_append", _append_writes_from_slot_zero),
    "append_mask_excludes_self": ("prefill_append", _append_mask_excludes_self),
    "rope_wrong_sign": ("rope_rotate_half", _rope_sign),
    "rope_frequency_exponent": ("rope_frequencies", _freq_exponent),
    "rmsnorm_eps_outside_sqrt": ("rms_norm", _eps_outside),
    "rmsnorm_weight_dropped": ("rms_norm", _no_weight),
    "rmsnorm_mean_centred": ("rms_norm", _mean_not_rms),
    "scale_one_over_d": ("causal_gqa_attention", _scale_one_over_d),
    "gqa_modulo_mapping": ("causal_gqa_attention", _gqa_modulo),
    "mask_off_by_one": ("causal_gqa_attention", _mask_sees_next),
    "k_v_columns_swapped": ("split_qkv", _kv_swapped),
    "v_normalised": ("qk_norm_rope", _v_normalised),
    "decode_skips_new_token": ("attend_prefix", _decode_without_self),
    "softmax_not_normalised": ("softmax", _softmax_no_norm),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(orc)
        except Exception as exc:  # any failure (assertion, shape error) means the pin noticed
            caught.append((check.__name__, type(exc).__name__))
            break
    assert caught, f"mutant {name} passed every pin"


# ---- steps around the attention layer (oracle.layer_ops) ----------------------

LO_REAL = {name: getattr(lo, name) for name in ("fused_add_rms_norm", "last_positions", "greedy_argmax")}


def _fused_residual_not_updated(x, residual, weight, eps):
    out, r = LO_REAL["fused_add_rms_norm"](x, residual, weight, eps)
    return out, (np.asarray(x, dtype=np.float64) if residual is None else np.asarray(residual, dtype=np.float64))


def _fused_normalises_x(x, residual, weight, eps):
    _, r = LO_REAL["fused_add_rms_norm"](x, residual, weight, eps)
    return orc.rms_norm(x, weight, eps), r


def _fused_adds_after_norm(x, residual, weight, eps):
    if residual is None:
        return LO_REAL["fused_add_rms_norm"](x, residual, weight, eps)
    r = np.asarray(x, dtype=np.float64) + np.asarray(residual, dtype=np.float64)
    return orc.rms_norm(x, weight, eps) + np.asarray(residual, dtype=np.float64), r


def _first_position(cu_seqlens):
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    return np.array([cu[r] if cu[r + 1] > cu[r] else -1 for r in range(len(cu) - 1)], dtype=np.int64)


def _argmax_last_tie(logits):
    z = np.asarray(logits, dtype=np.float64)[:, ::-1]
    return z.shape[1] - 1 - LO_REAL["greedy_argmax"](z)


def _argmax_ignores_nan(logits):
    z = np.asarray(logits, dtype=np.float64)
    return LO_REAL["greedy_argmax"](np.where(np.isnan(z), -np.inf, z))


LO_MUTANTS = {
    "fused_residual_not_updated": ("fused_add_rms_norm", _fused_residual_not_updated),
    "fused_normalises_x_not_sum": ("fused_add_rms_norm", _fused_normalises_x),
    "fused_adds_after_norm": ("fused_add_rms_norm", _fused_adds_after_norm),
    "gather_first_position": ("last_positions", _first_position),
    "argmax_last_tie": ("greedy_argmax", _argmax_last_tie),
    "argmax_ignores_nan": ("greedy_argmax", _argmax_ignores_nan),
}


@pytest.mark.parametrize("name", sorted(LO_MUTANTS))
def test_planted_layer_ops_mistake_is_caught(name, monkeypatch):
    attr, fn = LO_MUTANTS[name]
    monkeypatch.setattr(lo, attr, fn)
    caught = []
    for check in pins.LAYER_OPS_CHECKS:
        try:
            check(lo)
        except Exception as exc:
            caught.append((check.__name__, type(exc).__name__))
            break
    assert caught, f"mutant {name} passed every pin"


# ---- paged cache (oracle/paged.py) -------------------------------------------
import oracle.paged as pg  # noqa: E402

PG_REAL = {name: getattr(pg, name) for name in ("page_of", "scatter", "gather")}


def _page_and_row_swapped(table, b, s, page_size):
    return int(np.asarray(table)[b, s % page_size]), s // page_size


def _first_request_table(table, b, s, page_size):
    return int(np.asarray(table)[0, s // page_size]), s % page_size


def _next_page(table, b, s, page_size):
    t = np.asarray(table)
    return int(t[b, (s // page_size + 1) % t.shape[1]]), s % page_size


def _scatter_one_slot_late(pool, table, request, slots, values, page_size):
    return PG_REAL["scatter"](pool, table, request, [int(s) + 1 for s in slots], values, page_size)


def _gather_reversed_rows(pool, table, request, num_slots, page_size):
    out = PG_REAL["gather"](pool, table, request, num_slots, page_size)
    return out[:, ::-1, :].copy()


PG_MUTANTS = {
    "page_and_row_swapped": ("page_of", _page_and_row_swapped),
    "table_of_request_0": ("page_of", _first_request_table),
    "next_page": ("page_of", _next_page),
    "scatter_one_slot_late": ("scatter", _scatter_one_slot_late),
    "gather_reversed": ("gather", _gather_reversed_rows),
}


@pytest.mark.parametrize("name", sorted(PG_MUTANTS))
def test_planted_paged_mistake_is_caught(name, monkeypatch):
    attr, fn = PG_MUTANTS[name]
    monkeypatch.setattr(pg, attr, fn)
    caught = []
    for check in pins.PAGED_CHECKS:
        try:
            check(pg)
        except Exception as exc:
            caught.append((check.__name__, type(exc).__name__))
            break
    assert caught, f"mutant {name} passed every pin"
