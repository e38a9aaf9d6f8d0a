"""Checks that pin the oracle to facts outside itself.

Each ``check_*`` takes the oracle module and raises ``AssertionError`` when
the oracle disagrees with a closed form, an invariant the pages state, an
independent evaluator or a printed shape.  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutations.py`` runs them on deliberately broken
copies of oracle functions and expects each copy to fail at least one check.
"""

from __future__ import annotations

import json
import math
import pathlib

import numpy as np
import torch

import evaluators

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _layer_args(hq, hkv, d, eps=1e-6, base=1e4):
    return dict(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, rms_eps=eps, rope_base=base)


def _random_prefill(orc, seqlens, hq, hkv, d, seed, base=1e4, eps=1e-6, qkv=None):
    r = _rng(seed)
    n = int(sum(seqlens))
    width = (hq + 2 * hkv) * d
    if qkv is None:
        qkv = r.standard_normal((n, width))
    wq = 1 + 0.1 * r.standard_normal(d)
    wk = 1 + 0.1 * r.standard_normal(d)
    pos = np.concatenate([np.arange(t) for t in seqlens]) if seqlens else np.zeros(0)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    res = orc.prefill(qkv, wq, wk, pos, cu, cache_capacity=max(seqlens), **_layer_args(hq, hkv, d, eps, base))
    return qkv, wq, wk, pos, cu, res


# ---------------------------------------------------------------------------
# Split (column layout of the packed projection)
# ---------------------------------------------------------------------------

def check_split_layout(orc):
    hq, hkv, d = 4, 2, 3
    width = (hq + 2 * hkv) * d
    # Column c of the packed row holds the value c: Q heads, then K, then V.
    qkv = np.tile(np.arange(width, dtype=np.float64), (2, 1))
    q, k, v = orc.split_qkv(qkv, hq, hkv, d)
    assert q.shape == (2, hq, d) and k.shape == (2, hkv, d) and v.shape == (2, hkv, d)
    for h in range(hq):
        assert list(q[1, h]) == [h * d + e for e in range(d)]
    for g in range(hkv):
        assert list(k[0, g]) == [(hq + g) * d + e for e in range(d)]
        assert list(v[0, g]) == [(hq + hkv + g) * d + e for e in range(d)]


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def check_rmsnorm_constant_vector(orc):
    d, c, eps = 16, 0.37, 1e-2
    w = 1 + 0.1 * _rng(1).standard_normal(d)
    got = orc.rms_norm(np.full((1, d), c), w, eps)
    want = c / math.sqrt(c * c + eps) * w
    np.testing.assert_allclose(got[0], want, rtol=1e-14, atol=0)


def check_rmsnorm_library(orc):
    # torch.nn.functional.rms_norm: x * rsqrt(mean(x^2) + eps) * weight.
    r = _rng(2)
    x = r.standard_normal((5, 3, 32)) * 3
    w = 1 + 0.1 * r.standard_normal(32)
    for eps in (1e-6, 0.5):
        want = torch.nn.functional.rms_norm(torch.from_numpy(x), (32,), torch.from_numpy(w), eps).numpy()
        np.testing.assert_allclose(orc.rms_norm(x, w, eps), want, rtol=1e-13, atol=1e-14)


def check_rmsnorm_unit_rms(orc):
    x = _rng(3).standard_normal((7, 64)) * 5
    y = orc.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    # Scale invariance when eps = 0.
    np.testing.assert_allclose(orc.rms_norm(2.5 * x, np.ones(64), 0.0), y, rtol=1e-13)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def check_rope_d2_rotation(orc):
    # D = 2: theta_0 = base^0 = 1, so position p turns (x0, x1) by p radians.
    x = np.array([[[0.6, -1.3]]])
    for p in (0, 1, 7, 1234):
        y = orc.rope_rotate_half(x, np.array([p]), 1e4)[0, 0]
        c, s = math.cos(p), math.sin(p)
        np.testing.assert_allclose(y, [0.6 * c + 1.3 * s, -1.3 * c + 0.6 * s], rtol=0, atol=1e-12)


def check_rope_d4_frequencies(orc):
    # D = 4, base 1e4: theta = (1, 1e4^(-1/2) = 0.01).  Unit vectors pick out
    # each pair's angle.
    p = 100
    e0 = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    e1 = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    y0 = orc.rope_rotate_half(e0, np.array([p]), 1e4)[0, 0]
    y1 = orc.rope_rotate_half(e1, np.array([p]), 1e4)[0, 0]
    np.testing.assert_allclose(y0, [math.cos(100.0), 0, math.sin(100.0), 0], atol=1e-12)
    np.testing.assert_allclose(y1, [0, math.cos(1.0), 0, math.sin(1.0)], atol=1e-12)


def check_rope_complex_form(orc):
    # Rotate-half RoPE is multiplication of z_i = x_i + i x_{i+D/2} by
    # exp(i p theta_i), theta_i = base^(-2i/D) (RoFormer).
    r = _rng(4)
    d, base = 64, 1e6
    x = r.standard_normal((9, 3, d))
    pos = np.array([0, 1, 2, 5, 100, 4095, 4096, 32767, 77])
    theta = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    want = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(orc.rope_rotate_half(x, pos, base), want, rtol=0, atol=1e-11)


def check_rope_norm_and_relativity(orc):
    r = _rng(5)
    d = 128
    q = r.standard_normal((1, 1, d))
    k = r.standard_normal((1, 1, d))
    for base in (1e4, 1e6):
        qm = orc.rope_rotate_half(q, np.array([37]), base)
        np.testing.assert_allclose(np.linalg.norm(qm), np.linalg.norm(q), rtol=1e-13)
        dots = []
        for shift in (0, 5, 1000):
            a = orc.rope_rotate_half(q, np.array([37 + shift]), base)
            b = orc.rope_rotate_half(k, np.array([12 + shift]), base)
            dots.append(float(np.sum(a * b)))
        np.testing.assert_allclose(dots, dots[0], rtol=1e-11)
        # Position 0 is the identity.
        assert np.array_equal(orc.rope_rotate_half(q, np.array([0]), base), q)


# ---------------------------------------------------------------------------
# Attention against independent evaluators
# ---------------------------------------------------------------------------

def _attn_case(seed, t, hq, hkv, d):
    r = _rng(seed)
    return r.standard_normal((t, hq, d)), r.standard_normal((t, hkv, d)), r.standard_normal((t, hkv, d))


def _teaching_layout(x):
    return torch.from_numpy(np.ascontiguousarray(np.transpose(x, (1, 0, 2))))[None]


def check_attention_vs_definition(orc):
    for seed, (t, hq, hkv, d) in enumerate([(1, 4, 2, 8), (3, 4, 2, 8), (17, 8, 2, 16), (40, 6, 3, 32),
                                            (33, 4, 4, 16), (9, 8, 1, 8)]):
        q, k, v = _attn_case(10 + seed, t, hq, hkv, d)
        out, probs = orc.causal_gqa_attention(q, k, v, return_probs=True)
        want, want_p = evaluators.grouped_attention(_teaching_layout(q), _teaching_layout(k), _teaching_layout(v))
        np.testing.assert_allclose(out, want[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(probs, want_p[0].numpy(), rtol=0, atol=1e-12)


def check_attention_vs_library(orc):
    for seed, (t, hq, hkv, d) in enumerate([(5, 4, 2, 8), (64, 4, 2, 64), (130, 16, 8, 32), (31, 32, 8, 16)]):
        q, k, v = _attn_case(20 + seed, t, hq, hkv, d)
        out = orc.causal_gqa_attention(q, k, v, block=48)
        for native in (False, True):
            want = evaluators.library_attention(_teaching_layout(q), _teaching_layout(k), _teaching_layout(v), native)
            np.testing.assert_allclose(out, want[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def check_layer_brute_force(orc):
    cases = [([3], 4, 2, 8, 1e4), ([1, 4], 2, 1, 4, 1e6), ([8], 4, 2, 16, 1e4), ([2, 0, 5], 4, 4, 8, 10.0)]
    for seed, (seqlens, hq, hkv, d, base) in enumerate(cases):
        qkv, wq, wk, pos, cu, res = _random_prefill(orc, seqlens, hq, hkv, d, 30 + seed, base=base, eps=1e-3)
        want = evaluators.brute_force_layer(qkv.tolist(), wq.tolist(), wk.tolist(), pos.tolist(), seqlens,
                                            hq, hkv, d, 1e-3, base)
        got = res["out"].reshape(-1, hq, d)
        np.testing.assert_allclose(got, np.array(want).reshape(got.shape), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms and invariants the pages state
# ---------------------------------------------------------------------------

def check_single_token_returns_v(orc):
    # T = 1: the only visible key is the token itself, so p = 1 and o_h = v_{h//G}.
    for hq, hkv in [(4, 2), (8, 8), (6, 1)]:
        qkv, wq, wk, pos, cu, res = _random_prefill(orc, [1, 1], hq, hkv, 8, 40)
        _, _, v = orc.split_qkv(qkv, hq, hkv, 8)
        out = res["out"].reshape(2, hq, 8)
        for h in range(hq):
            np.testing.assert_allclose(out[:, h], v[:, h // (hq // hkv)], rtol=0, atol=1e-14)


def check_zero_query_prefix_mean(orc):
    # Zero Q rows normalise to zero, every score is zero, so row i is the mean
    # of v_0..v_i of its KV head.
    hq, hkv, d, t = 4, 2, 8, 11
    r = _rng(41)
    qkv = r.standard_normal((t, (hq + 2 * hkv) * d))
    qkv[:, : hq * d] = 0.0
    _, _, _, _, _, res = _random_prefill(orc, [t], hq, hkv, d, 41, qkv=qkv)
    _, _, v = orc.split_qkv(qkv, hq, hkv, d)
    out = res["out"].reshape(t, hq, d)
    for h in range(hq):
        g = h // (hq // hkv)
        want = np.cumsum(v[:, g], axis=0) / np.arange(1, t + 1)[:, None]
        np.testing.assert_allclose(out[:, h], want, rtol=0, atol=1e-13)


def check_softmax_rows(orc):
    q, k, v = _attn_case(42, 13, 4, 2, 16)
    _, probs = orc.causal_gqa_attention(q, k, v, return_probs=True)
    np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=0, atol=1e-14)
    future = np.triu(np.ones((13, 13), dtype=bool), 1)
    assert np.all(probs[:, future] == 0.0)
    assert np.all(probs[:, ~future] > 0.0)


def check_causality(orc):
    hq, hkv, d, t = 4, 2, 16, 20
    qkv, wq, wk, pos, cu, res = _random_prefill(orc, [t], hq, hkv, d, 43)
    for i in (0, 7, 18):
        changed = qkv.copy()
        changed[i + 1:] = _rng(44 + i).standard_normal(changed[i + 1:].shape)
        res2 = orc.prefill(changed, wq, wk, pos, cu, cache_capacity=t, **_layer_args(hq, hkv, d))
        assert np.array_equal(res2["out"][: i + 1], res["out"][: i + 1])
        assert not np.allclose(res2["out"][i + 1:], res["out"][i + 1:])


def check_request_isolation(orc):
    hq, hkv, d = 4, 2, 8
    seqlens = [5, 9, 3]
    qkv, wq, wk, pos, cu, res = _random_prefill(orc, seqlens, hq, hkv, d, 45)
    changed = qkv.copy()
    changed[5:14] = _rng(46).standard_normal((9, qkv.shape[1]))
    res2 = orc.prefill(changed, wq, wk, pos, cu, cache_capacity=9, **_layer_args(hq, hkv, d))
    np.testing.assert_array_equal(res2["out"][:5], res["out"][:5])
    np.testing.assert_array_equal(res2["out"][14:], res["out"][14:])
    # Each request alone gives the same rows as the packed batch.
    for r in range(3):
        lo, hi = int(cu[r]), int(cu[r + 1])
        alone = orc.prefill(qkv[lo:hi], wq, wk, pos[lo:hi], [0, hi - lo], cache_capacity=hi - lo,
                            **_layer_args(hq, hkv, d))
        np.testing.assert_allclose(alone["out"], res["out"][lo:hi], rtol=0, atol=1e-14)


def check_gqa_grouping(orc):
    # Repeating each KV head G times in a row (so Hkv becomes Hq) gives the
    # same output as reading KV head h // G; with Hq=4, Hkv=2 this differs
    # from reading h % Hkv.
    q, k, v = _attn_case(47, 9, 4, 2, 8)
    grouped = orc.causal_gqa_attention(q, k, v)
    repeated = orc.causal_gqa_attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1))
    np.testing.assert_allclose(grouped, repeated, rtol=0, atol=1e-15)
    modulo = orc.causal_gqa_attention(q, np.tile(k, (1, 2, 1)), np.tile(v, (1, 2, 1)))
    assert not np.allclose(grouped, modulo)


def check_prefill_cache_layout(orc):
    hq, hkv, d = 4, 2, 8
    seqlens = [3, 0, 5]
    qkv, wq, wk, pos, cu, res = _random_prefill(orc, seqlens, hq, hkv, d, 48)
    q_t, k_t, v = orc.qk_norm_rope(qkv, wq, wk, pos, **_layer_args(hq, hkv, d))
    _, _, v_raw = orc.split_qkv(qkv, hq, hkv, d)
    kc, vc = res["k_cache"], res["v_cache"]
    assert kc.shape == (3, hkv, 5, d)
    for r, (lo, t) in enumerate(zip(cu[:-1], seqlens)):
        for j in range(5):
            if j < t:
                np.testing.assert_array_equal(vc[r, :, j], v_raw[lo + j])
                np.testing.assert_allclose(kc[r, :, j], k_t[lo + j], rtol=0, atol=0)
            else:
                assert np.all(np.isnan(kc[r, :, j])) and np.all(np.isnan(vc[r, :, j]))


def check_decode_is_last_prefill_row(orc):
    # A decode step over a cache of L entries equals row L of a prefill over
    # the L+1 tokens (the cache grows by one, then the new row attends).
    hq, hkv, d = 8, 2, 16
    for seed, length in enumerate([0, 1, 6, 21]):
        t = length + 1
        qkv, wq, wk, pos, cu, res = _random_prefill(orc, [t], hq, hkv, d, 50 + seed)
        cap = t + 2
        kc = np.full((1, hkv, cap, d), np.nan)
        vc = np.full((1, hkv, cap, d), np.nan)
        kc[0, :, :length] = res["k_cache"][0, :, :length]
        vc[0, :, :length] = res["v_cache"][0, :, :length]
        dec = orc.decode(qkv[length:], wq, wk, [length], [length], kc, vc, **_layer_args(hq, hkv, d))
        np.testing.assert_allclose(dec["out"][0], res["out"][length], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dec["k_cache"][0, :, : t], res["k_cache"][0, :, : t], rtol=0, atol=1e-15)
        np.testing.assert_array_equal(dec["v_cache"][0, :, : t], res["v_cache"][0, :, : t])
        assert np.all(np.isnan(dec["k_cache"][0, :, t:]))


def check_sampled_rows(orc):
    hq, hkv, d = 4, 2, 8
    seqlens = [7, 12]
    qkv, wq, wk, pos, cu, res = _random_prefill(orc, seqlens, hq, hkv, d, 55)
    rows = orc.prefill_rows(res["q_tilde"], res["k_tilde"], res["v"], cu, [0, 6, 7, 13, 18])
    full = res["out"].reshape(-1, hq, d)
    for n, row in rows.items():
        np.testing.assert_allclose(row, full[n], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# Appending a chunk to a filled cache: it contains prefill (empty cache) and
# decode (one-token chunks), and a prefill split in two equals the whole.
# ---------------------------------------------------------------------------

def _append_on(orc, qkv, wq, wk, pos, cu, lens, kc, vc, hq, hkv, d, base=1e4, eps=1e-6):
    return orc.prefill_append(qkv, wq, wk, pos, cu, lens, kc, vc, **_layer_args(hq, hkv, d, eps, base))


def check_append_to_empty_cache_is_prefill(orc):
    hq, hkv, d = 4, 2, 8
    seqlens = [5, 0, 9, 1]
    qkv, wq, wk, pos, cu, res = _random_prefill(orc, seqlens, hq, hkv, d, 60)
    shape = (len(seqlens), hkv, max(seqlens), d)
    got = _append_on(orc, qkv, wq, wk, pos, cu, [0] * len(seqlens), np.full(shape, np.nan), np.full(shape, np.nan),
                     hq, hkv, d)
    np.testing.assert_allclose(got["out"], res["out"], rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isnan(got["k_cache"]), np.isnan(res["k_cache"]))
    np.testing.assert_allclose(np.nan_to_num(got["k_cache"]), np.nan_to_num(res["k_cache"]), rtol=0, atol=1e-15)


def check_append_single_tokens_is_decode(orc):
    hq, hkv, d = 8, 2, 16
    r = _rng(61)
    lens = [0, 3, 17]
    cap = 20
    kc = r.standard_normal((3, hkv, cap, d))
    vc = r.standard_normal((3, hkv, cap, d))
    qkv = r.standard_normal((3, (hq + 2 * hkv) * d))
    wq = 1 + 0.1 * r.standard_normal(d)
    wk = 1 + 0.1 * r.standard_normal(d)
    dec = orc.decode(qkv, wq, wk, lens, lens, kc, vc, **_layer_args(hq, hkv, d))
    got = _append_on(orc, qkv, wq, wk, lens, [0, 1, 2, 3], lens, kc, vc, hq, hkv, d)
    np.testing.assert_allclose(got["out"], dec["out"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(got["k_cache"], dec["k_cache"], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(got["v_cache"], dec["v_cache"])


def check_append_split_equals_full_prefill(orc):
    # Prefill of the first T1 tokens, then the next T2 appended onto that
    # cache, gives the last T2 rows (and the cache) of a prefill of T1 + T2.
    hq, hkv, d = 4, 2, 16
    splits = [(3, 4), (0, 6), (7, 0), (1, 1), (9, 5)]
    full_lens = [a + b for a, b in splits]
    qkv, wq, wk, pos, cu, res = _random_prefill(orc, full_lens, hq, hkv, d, 62, base=1e6)
    cap = max(full_lens) + 2
    b = len(splits)
    kc = np.full((b, hkv, cap, d), np.nan)
    vc = np.full((b, hkv, cap, d), np.nan)
    rows, cu2 = [], [0]
    for i, (t1, t2) in enumerate(splits):
        kc[i, :, :t1] = res["k_cache"][i, :, :t1]
        vc[i, :, :t1] = res["v_cache"][i, :, :t1]
        rows.extend(range(cu[i] + t1, cu[i] + t1 + t2))
        cu2.append(cu2[-1] + t2)
    got = _append_on(orc, qkv[rows], wq, wk, pos[rows], cu2, [t1 for t1, _ in splits], kc, vc, hq, hkv, d,
                     base=1e6)
    np.testing.assert_allclose(got["out"], res["out"][rows], rtol=0, atol=1e-13)
    for i, n in enumerate(full_lens):
        np.testing.assert_allclose(got["k_cache"][i, :, :n], res["k_cache"][i, :, :n], rtol=0, atol=1e-15)
        np.testing.assert_array_equal(got["v_cache"][i, :, :n], res["v_cache"][i, :, :n])
        assert np.all(np.isnan(got["k_cache"][i, :, n:]))


def check_append_brute_force(orc):
    # Scalar loops over the whole sequence (history and chunk) at tiny sizes.
    hq, hkv, d = 4, 2, 8
    t1, t2 = 3, 4
    r = _rng(63)
    n = t1 + t2
    qkv = r.standard_normal((n, (hq + 2 * hkv) * d))
    wq = 1 + 0.1 * r.standard_normal(d)
    wk = 1 + 0.1 * r.standard_normal(d)
    pos = np.arange(n)
    pre = orc.prefill(qkv[:t1], wq, wk, pos[:t1], [0, t1], cache_capacity=n, **_layer_args(hq, hkv, d, 1e-3))
    got = _append_on(orc, qkv[t1:], wq, wk, pos[t1:], [0, t2], [t1], pre["k_cache"], pre["v_cache"], hq, hkv, d,
                     eps=1e-3)
    want = evaluators.brute_force_layer(qkv.tolist(), wq.tolist(), wk.tolist(), pos.tolist(), [n], hq, hkv, d,
                                        1e-3, 1e4)
    np.testing.assert_allclose(got["out"].reshape(t2, hq, d), np.array(want)[t1:], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Shapes and cache lengths the pages print
# ---------------------------------------------------------------------------

def check_golden_shapes(orc):
    fx = json.loads((GOLDEN / "shapes_walkthrough_sec5.json").read_text())
    t, hq, hkv, d = fx["T"], fx["Hq"], fx["Hkv"], fx["D"]
    qkv, wq, wk, pos, cu, res = _random_prefill(orc, [t], hq, hkv, d, 60)
    q, k, v = orc.split_qkv(qkv, hq, hkv, d)
    assert [1] + list(np.transpose(q, (1, 0, 2)).shape) == fx["q_shape"]
    assert [1] + list(np.transpose(k, (1, 0, 2)).shape) == fx["kv_shape"]
    _, probs = orc.causal_gqa_attention(res["q_tilde"], res["k_tilde"], res["v"], return_probs=True)
    assert [1] + list(probs.shape) == fx["scores_shape"]

    fx = json.loads((GOLDEN / "shapes_qwen3_4b_prefill.json").read_text())
    t, hq, hkv, d = fx["T"], fx["Hq"], fx["Hkv"], fx["D"]
    r = _rng(61)
    qkv = r.standard_normal((t, (hq + 2 * hkv) * d))
    q, k, v = orc.split_qkv(qkv, hq, hkv, d)
    assert [1, t, q.shape[1] * d] == fx["q_proj"] and [1, t, k.shape[1] * d] == fx["kv_proj"]
    assert [1] + list(q.shape) == fx["q_view"] and [1] + list(k.shape) == fx["kv_view"]
    res = orc.prefill(qkv, np.ones(d), np.ones(d), np.arange(t), [0, t], cache_capacity=t + 1,
                      **_layer_args(hq, hkv, d, base=1e6))
    _, probs = orc.causal_gqa_attention(res["q_tilde"], res["k_tilde"], res["v"], return_probs=True)
    assert [1] + list(probs.shape) == fx["attn_weights"]
    assert [1] + list(res["out"].shape) == fx["attn_output_flat"]


def check_golden_cache_lengths(orc):
    fx = json.loads((GOLDEN / "cache_lengths_prefill_decode.json").read_text())
    hq, hkv, d = 4, 2, 8
    t = fx["prompt_tokens"]
    qkv, wq, wk, pos, cu, res = _random_prefill(orc, [t], hq, hkv, d, 62)

    def filled(cache):
        return int(np.sum(~np.isnan(cache[0, 0, :, 0])))

    assert filled(np.full((1, hkv, t + 1, d), np.nan)) == fx["before_prefill"]
    kc = np.full((1, hkv, t + 1, d), np.nan)
    kc[:, :, :t] = res["k_cache"]
    vc = np.full((1, hkv, t + 1, d), np.nan)
    vc[:, :, :t] = res["v_cache"]
    assert filled(kc) == fx["after_prefill"] == fx["decode_before_update"]
    row = _rng(63).standard_normal((1, qkv.shape[1]))
    dec = orc.decode(row, wq, wk, [t], [t], kc, vc, **_layer_args(hq, hkv, d))
    assert filled(dec["k_cache"]) == filled(dec["v_cache"]) == fx["decode_after_update"]


ALL_CHECKS = [
    check_split_layout,
    check_rmsnorm_constant_vector,
    check_rmsnorm_library,
    check_rmsnorm_unit_rms,
    check_rope_d2_rotation,
    check_rope_d4_frequencies,
    check_rope_complex_form,
    check_rope_norm_and_relativity,
    check_attention_vs_definition,
    check_attention_vs_library,
    check_layer_brute_force,
    check_single_token_returns_v,
    check_zero_query_prefix_mean,
    check_softmax_rows,
    check_causality,
    check_request_isolation,
    check_gqa_grouping,
    check_prefill_cache_layout,
    check_decode_is_last_prefill_row,
    check_sampled_rows,
    check_golden_shapes,
    check_golden_cache_lengths,
    check_append_to_empty_cache_is_prefill,
    check_append_single_tokens_is_decode,
    check_append_split_equals_full_prefill,
    check_append_brute_force,
]


# ---------------------------------------------------------------------------
# Steps around the attention layer (oracle.layer_ops): the fused residual add
# + RMSNorm (Code Walkthrough, section 3.2) and next-token selection (section
# 4.1: each request's last row; section 4.3: greedy argmax).  These checks take
# the ``oracle.layer_ops`` module.
# ---------------------------------------------------------------------------

def _torch_rms_norm(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return torch.nn.functional.rms_norm(torch.from_numpy(x), (x.shape[-1],),
                                        torch.from_numpy(np.asarray(w, dtype=np.float64)), eps).numpy()


def check_fused_norm_first_call(lo):
    # No residual yet: x itself becomes the residual and the output is RMSNorm(x).
    r = _rng(80)
    x = r.standard_normal((6, 48)) * 2
    w = 1 + 0.1 * r.standard_normal(48)
    out, res = lo.fused_add_rms_norm(x, None, w, 1e-6)
    assert np.array_equal(res, x)
    np.testing.assert_allclose(out, _torch_rms_norm(x, w, 1e-6), rtol=1e-13, atol=1e-14)


def check_fused_norm_adds_then_normalises(lo):
    # Integer-valued inputs, so the sum is exact and known: the new residual is
    # x + residual; the output is the library RMSNorm of that sum.
    r = _rng(81)
    x = r.integers(-8, 9, (5, 40)).astype(np.float64)
    res0 = r.integers(-8, 9, (5, 40)).astype(np.float64)
    w = 1 + 0.1 * r.standard_normal(40)
    out, res = lo.fused_add_rms_norm(x, res0, w, 1e-6)
    total = np.array([[int(a) + int(b) for a, b in zip(ra, rb)] for ra, rb in zip(x, res0)], dtype=np.float64)
    assert np.array_equal(res, total)
    np.testing.assert_allclose(out, _torch_rms_norm(total, w, 1e-6), rtol=1e-13, atol=1e-14)


def check_fused_norm_constant_rows(lo):
    # x = a*1 and residual = b*1: the output is (a+b)/sqrt((a+b)^2 + eps) * w.
    c, eps = 24, 1e-2
    w = 1 + 0.1 * _rng(82).standard_normal(c)
    for a, b in ((0.25, 0.5), (-1.5, 0.25), (2.0, -2.0)):
        out, res = lo.fused_add_rms_norm(np.full((1, c), a), np.full((1, c), b), w, eps)
        s = a + b
        np.testing.assert_allclose(res[0], s, rtol=0, atol=0)
        np.testing.assert_allclose(out[0], s / math.sqrt(s * s + eps) * w, rtol=1e-14, atol=1e-15)


def check_fused_norm_decoder_chain(lo):
    # The pages' layer loop, written with the fused call, equals the expanded
    # form h = x + Attn(RMSNorm(x)), out = h + MLP(RMSNorm(h)) followed by the
    # model's final norm (section 3.2).  The sublayers are fixed stand-ins.
    r = _rng(83)
    n, c, layers, eps = 5, 32, 3, 1e-6
    x0 = r.standard_normal((n, c))
    w_in = [1 + 0.1 * r.standard_normal(c) for _ in range(layers)]
    w_post = [1 + 0.1 * r.standard_normal(c) for _ in range(layers)]
    w_final = 1 + 0.1 * r.standard_normal(c)
    attn = [r.standard_normal((c, c)) / math.sqrt(c) for _ in range(layers)]
    mlp = [r.standard_normal((c, c)) / math.sqrt(c) for _ in range(layers)]
    x, res = x0, None
    for i in range(layers):
        x, res = lo.fused_add_rms_norm(x, res, w_in[i], eps)
        x = np.tanh(x @ attn[i])
        x, res = lo.fused_add_rms_norm(x, res, w_post[i], eps)
        x = np.tanh(x @ mlp[i])
    got, _ = lo.fused_add_rms_norm(x, res, w_final, eps)
    h = x0
    for i in range(layers):
        h = h + np.tanh(_torch_rms_norm(h, w_in[i], eps) @ attn[i])
        h = h + np.tanh(_torch_rms_norm(h, w_post[i], eps) @ mlp[i])
    np.testing.assert_allclose(got, _torch_rms_norm(h, w_final, eps), rtol=1e-12, atol=1e-12)


def check_last_positions_pages_example(lo):
    # Section 4.1: for the input [1, 2, 3] the logits at position 2 predict the
    # next token, so a 3-token request selects row 2.  Packed requests select
    # cu[r+1]-1; an empty request selects nothing (-1).
    assert list(lo.last_positions([0, 3])) == [2]
    assert list(lo.last_positions([0, 3, 3, 7, 8])) == [2, -1, 6, 7]


def check_gather_last_rows(lo):
    h = _rng(84).standard_normal((8, 6))
    g = lo.gather_last(h, [0, 3, 3, 7, 8])
    assert np.array_equal(g[0], h[2]) and np.array_equal(g[2], h[6]) and np.array_equal(g[3], h[7])
    assert np.isnan(g[1]).all()


def check_argmax_library(lo):
    # Rows without ties: numpy's and torch's argmax.
    z = _rng(85).standard_normal((7, 300))
    got = lo.greedy_argmax(z)
    assert np.array_equal(got, np.argmax(z, axis=1))
    assert np.array_equal(got, torch.argmax(torch.from_numpy(z), dim=-1).numpy())


def check_argmax_ties_and_nan(lo):
    # Ties go to the lowest index; a NaN beats every number (first NaN wins).
    z = np.zeros((5, 10))
    z[0, [3, 7]] = 5.0
    z[2, 4], z[2, 8] = np.nan, 100.0
    z[3, [6, 2]] = np.nan
    z[4] = -np.inf
    z[4, 9] = -1e300
    assert list(lo.greedy_argmax(z)) == [3, 0, 4, 2, 9]
    assert list(np.argmax(z, axis=1)) == [3, 0, 4, 2, 9]


LAYER_OPS_CHECKS = [
    check_fused_norm_first_call,
    check_fused_norm_adds_then_normalises,
    check_fused_norm_constant_rows,
    check_fused_norm_decoder_chain,
    check_last_positions_pages_example,
    check_gather_last_rows,
    check_argmax_library,
    check_argmax_ties_and_nan,
]


# ---------------------------------------------------------------------------
# Paged K/V cache (oracle/paged.py).  The reading: a paged cache is the
# per-request cache with its slots stored in pages of a pool, found through a
# block table; every result is the contiguous cache's.  These checks pin the
# paged oracle to the flat-address formula written out here, to the already
# pinned contiguous oracle, and to scalar brute force of the whole layer over
# the tokens (which knows nothing about pages).
# ---------------------------------------------------------------------------

def _shuffled_table(r, num_seqs, pages_per_seq, num_pages):
    """Distinct random pages for every (request, page index); the unused pages of the pool are holes."""
    assert num_pages >= num_seqs * pages_per_seq
    return r.permutation(num_pages)[: num_seqs * pages_per_seq].reshape(num_seqs, pages_per_seq)


def check_paged_flat_address(pg):
    # Element (b, g, s, d) of the logical cache sits at ((table[b][s // P] * Hkv + g) * P + s % P) * D + d of the
    # flat pool: scatter then gather through the oracle agree with that formula written out as scalar loops.
    r = _rng(70)
    hkv, d, page, num_pages = 2, 3, 4, 13
    table = _shuffled_table(r, 3, 3, num_pages)
    lens = [5, 12, 0]
    flat = np.full(num_pages * hkv * page * d, np.nan)
    pool = np.full((num_pages, hkv, page, d), np.nan)
    for b, n in enumerate(lens):
        vals = r.standard_normal((hkv, n, d))
        pg.scatter(pool, table, b, list(range(n)), vals, page)
        for s in range(n):
            for g in range(hkv):
                for e in range(d):
                    flat[((int(table[b, s // page]) * hkv + g) * page + s % page) * d + e] = vals[g, s, e]
        np.testing.assert_array_equal(pg.gather(pool, table, b, n, page), vals)
    np.testing.assert_array_equal(pool.reshape(-1), flat)  # NaN where no slot was written (the holes)


def _paged_layer(r, hq, hkv, d, base=1e4):
    return dict(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, rms_eps=1e-6, rope_base=base)


def check_paged_identity_table_is_contiguous(pg):
    # One page per request holding its whole cache (P = capacity, table[b] = [b]): the pool is the contiguous
    # cache [B, Hkv, S, D] itself, and both modes give the contiguous oracle's results bit for bit.
    import oracle.qknorm_rope_attn as orc

    r = _rng(71)
    hq, hkv, d, cap = 4, 2, 8, 9
    lens = [3, 0, 8]
    kc = r.standard_normal((3, hkv, cap, d))
    vc = r.standard_normal((3, hkv, cap, d))
    qkv = r.standard_normal((3, (hq + 2 * hkv) * d))
    wq, wk = 1 + 0.1 * r.standard_normal(d), 1 + 0.1 * r.standard_normal(d)
    table = np.arange(3).reshape(3, 1)
    got = pg.decode(qkv, wq, wk, lens, lens, kc, vc, table, cap, **_paged_layer(r, hq, hkv, d))
    want = orc.decode(qkv, wq, wk, lens, lens, kc, vc, **_paged_layer(r, hq, hkv, d))
    np.testing.assert_array_equal(got["out"], want["out"])
    np.testing.assert_array_equal(got["k_pool"], want["k_cache"])
    np.testing.assert_array_equal(got["v_pool"], want["v_cache"])
    chunks = [2, 1, 0]
    cu = np.concatenate([[0], np.cumsum(chunks)])
    rows = r.standard_normal((3, (hq + 2 * hkv) * d))
    pos = np.array([3, 4, 0])
    got = pg.prefill_append(rows, wq, wk, pos, cu, [3, 0, 8], kc, vc, table, cap, **_paged_layer(r, hq, hkv, d))
    want = orc.prefill_append(rows, wq, wk, pos, cu, [3, 0, 8], kc, vc, **_paged_layer(r, hq, hkv, d))
    np.testing.assert_array_equal(got["out"], want["out"])
    np.testing.assert_array_equal(got["k_pool"], want["k_cache"])


def check_paged_brute_force(pg):
    # Prefill through a shuffled table with holes, then one decode step per request: every output equals the
    # scalar brute force of the whole layer over the request's tokens (no pages involved).  Page sizes 1, 2, 3
    # put page boundaries everywhere; pages no request owns stay NaN.
    import evaluators

    for seed, (page, hq, hkv, d) in enumerate([(2, 4, 2, 8), (3, 2, 1, 4), (1, 4, 4, 8)]):
        r = _rng(72 + seed)
        seqlens = [5, 1, 4]
        cap_pages = (max(seqlens) + 1 + page - 1) // page
        num_pages = 3 * cap_pages + 5
        table = _shuffled_table(r, 3, cap_pages, num_pages)
        width = (hq + 2 * hkv) * d
        tokens = [r.standard_normal((t + 1, width)) for t in seqlens]  # the prompt and then the decoded token
        wq, wk = 1 + 0.1 * r.standard_normal(d), 1 + 0.1 * r.standard_normal(d)
        kp = np.full((num_pages, hkv, page, d), np.nan)
        vp = np.full((num_pages, hkv, page, d), np.nan)
        prompt = np.concatenate([x[:-1] for x in tokens])
        cu = np.concatenate([[0], np.cumsum(seqlens)])
        pos = np.concatenate([np.arange(t) for t in seqlens])
        pre = pg.prefill_append(prompt, wq, wk, pos, cu, [0, 0, 0], kp, vp, table, page, **_paged_layer(r, hq, hkv, d))
        dec = pg.decode(np.stack([x[-1] for x in tokens]), wq, wk, seqlens, seqlens, pre["k_pool"], pre["v_pool"],
                        table, page, **_paged_layer(r, hq, hkv, d))
        used = set(int(p) for p in table[:, :].reshape(-1))
        for p in range(num_pages):
            if p not in used:
                assert np.all(np.isnan(dec["k_pool"][p])) and np.all(np.isnan(dec["v_pool"][p])), f"hole {p} written"
        for b, t in enumerate(seqlens):
            want = evaluators.brute_force_layer(tokens[b].tolist(), wq.tolist(), wk.tolist(), list(range(t + 1)),
                                                [t + 1], hq, hkv, d, 1e-6, 1e4)
            want = np.array(want).reshape(t + 1, hq * d)
            np.testing.assert_allclose(pre["out"][cu[b]:cu[b + 1]], want[:t], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dec["out"][b], want[t], rtol=0, atol=1e-12)


def check_paged_page_permutation(pg):
    # Renaming the pool's pages (pool permuted, table mapped the same way) changes no result, and the written
    # pool is the permuted written pool.
    r = _rng(75)
    hq, hkv, d, page, num_pages = 4, 2, 8, 2, 11
    lens = [3, 6]
    table = _shuffled_table(r, 2, 4, num_pages)
    kp, vp = r.standard_normal((num_pages, hkv, page, d)), r.standard_normal((num_pages, hkv, page, d))
    qkv = r.standard_normal((2, (hq + 2 * hkv) * d))
    wq, wk = 1 + 0.1 * r.standard_normal(d), 1 + 0.1 * r.standard_normal(d)
    perm = r.permutation(num_pages)            # page p moves to perm[p]
    kq, vq = np.empty_like(kp), np.empty_like(vp)
    kq[perm], vq[perm] = kp, vp
    a = pg.decode(qkv, wq, wk, lens, lens, kp, vp, table, page, **_paged_layer(r, hq, hkv, d))
    b = pg.decode(qkv, wq, wk, lens, lens, kq, vq, perm[table], page, **_paged_layer(r, hq, hkv, d))
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["k_pool"], b["k_pool"][perm])
    np.testing.assert_array_equal(a["v_pool"], b["v_pool"][perm])


def check_paged_shared_prefix(pg):
    # Two requests whose tables share their first pages (a prefix cached once) read the same history: each
    # decode equals the contiguous decode over its own copy of that history.  Their new slots land in pages of
    # their own, and the shared pages are not written.
    import oracle.qknorm_rope_attn as orc

    r = _rng(76)
    hq, hkv, d, page = 4, 2, 8, 2
    L = 4                                      # two full shared pages, new token in page index 2
    table = np.array([[5, 1, 3], [5, 1, 0]])
    kp, vp = r.standard_normal((6, hkv, page, d)), r.standard_normal((6, hkv, page, d))
    qkv = r.standard_normal((2, (hq + 2 * hkv) * d))
    wq, wk = 1 + 0.1 * r.standard_normal(d), 1 + 0.1 * r.standard_normal(d)
    got = pg.decode(qkv, wq, wk, [L, L], [L, L], kp, vp, table, page, **_paged_layer(r, hq, hkv, d))
    hist_k = np.concatenate([kp[5], kp[1]], axis=1)   # slots 0..3 of either request
    hist_v = np.concatenate([vp[5], vp[1]], axis=1)
    for b in range(2):
        kc = np.concatenate([hist_k, np.zeros((hkv, 1, d))], axis=1)[None]
        vc = np.concatenate([hist_v, np.zeros((hkv, 1, d))], axis=1)[None]
        want = orc.decode(qkv[b:b + 1], wq, wk, [L], [L], kc, vc, **_paged_layer(r, hq, hkv, d))
        np.testing.assert_array_equal(got["out"][b], want["out"][0])
    np.testing.assert_array_equal(got["k_pool"][[5, 1]], kp[[5, 1]])
    assert not np.array_equal(got["k_pool"][3][:, 0], kp[3][:, 0]) and not np.array_equal(got["k_pool"][0][:, 0],
                                                                                           kp[0][:, 0])


def check_paged_chunks_equal_full_prefill(pg):
    # A prompt appended in two chunks through a shuffled table gives the rows of one contiguous prefill of the
    # whole prompt, and the pool read back through the table is that prefill's cache.
    import oracle.qknorm_rope_attn as orc

    r = _rng(77)
    hq, hkv, d, page, num_pages = 4, 2, 8, 3, 9
    t1, t2 = 4, 5
    qkv = r.standard_normal((t1 + t2, (hq + 2 * hkv) * d))
    wq, wk = 1 + 0.1 * r.standard_normal(d), 1 + 0.1 * r.standard_normal(d)
    table = _shuffled_table(r, 1, 3, num_pages)
    kp = np.full((num_pages, hkv, page, d), np.nan)
    vp = np.full((num_pages, hkv, page, d), np.nan)
    a = pg.prefill_append(qkv[:t1], wq, wk, np.arange(t1), [0, t1], [0], kp, vp, table, page,
                          **_paged_layer(r, hq, hkv, d))
    b = pg.prefill_append(qkv[t1:], wq, wk, np.arange(t1, t1 + t2), [0, t2], [t1], a["k_pool"], a["v_pool"], table,
                          page, **_paged_layer(r, hq, hkv, d))
    full = orc.prefill(qkv, wq, wk, np.arange(t1 + t2), [0, t1 + t2], cache_capacity=t1 + t2,
                       **_paged_layer(r, hq, hkv, d))
    np.testing.assert_allclose(np.concatenate([a["out"], b["out"]]), full["out"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(pg.gather(b["k_pool"], table, 0, t1 + t2, page), full["k_cache"][0], rtol=0, atol=0)
    np.testing.assert_array_equal(pg.gather(b["v_pool"], table, 0, t1 + t2, page), full["v_cache"][0])


PAGED_CHECKS = [
    check_paged_flat_address,
    check_paged_identity_table_is_contiguous,
    check_paged_brute_force,
    check_paged_page_permutation,
    check_paged_shared_prefix,
    check_paged_chunks_equal_full_prefill,
]
