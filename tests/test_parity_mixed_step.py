"""qknorm_rope_attn_mixed_step on the GPU: a prefill batch and a decode batch in one call.

It computes what qknorm_rope_attn_prefill followed by qknorm_rope_attn_decode computes. In bf16, for the
head groupings it supports, it runs the prefill attention and the decode split in one launch. The decode role
runs the same wavefronts over the same plan as the decode split, and the prefill role the same work items, so
every output and cache must equal the two separate calls bit for bit. Both halves are also compared with the
oracle directly: the decode output of every request and its new cache slots, the prefill output (every row, or
at least 512 sampled rows per head on the benchmark workload) and the prefill caches. Outputs start as NaN, so a
row that no workgroup wrote shows. Groupings outside the supported set (G = 3 here) and fp32 take the two calls
in turn.
"""

import numpy as np
import pytest
import torch

import decoder_attention_amd as da
import oracle
from harness import (assert_close, bits, cfg_of, check_decode_result, check_prefill_caches, f64, layer_kw, note,
                     oracle_prefill, sample_tokens, tol_for)
from workloads import HeadConfig, build_workload, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _both(p, d):
    """Separate calls on clones of the caches, then the mixed step on the originals; returns both results and the
    caches as they were before either call."""
    h = p.heads
    cfg = cfg_of(h, p.qkv.dtype)
    width = h.num_q_heads * h.head_dim
    pk, pv, dk, dv = p.k_cache.clone(), p.v_cache.clone(), d.k_cache.clone(), d.v_cache.clone()
    before = (p.k_cache.clone(), p.v_cache.clone(), d.k_cache.clone(), d.v_cache.clone())
    sep_p, _ = da.prefill(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens, p.max_seqlen,
                          pk, pv, out=_nan((p.num_tokens, width), p.qkv.dtype))
    sep_d, _ = da.decode(cfg, d.qkv, p.q_norm_weight, p.k_norm_weight, d.positions, d.cache_lens, d.max_cache_len,
                         dk, dv, out=_nan((d.num_seqs, width), d.qkv.dtype))
    mix_p, mix_d, _, _ = da.mixed_step(cfg, p.q_norm_weight, p.k_norm_weight, p.qkv, p.positions, p.cu_seqlens,
                                       p.max_seqlen, p.k_cache, p.v_cache, d.qkv, d.positions, d.cache_lens,
                                       d.max_cache_len, d.k_cache, d.v_cache,
                                       prefill_out=_nan((p.num_tokens, width), p.qkv.dtype),
                                       decode_out=_nan((d.num_seqs, width), d.qkv.dtype))
    torch.cuda.synchronize()
    return (sep_p, sep_d, pk, pv, dk, dv), (mix_p, mix_d, p.k_cache, p.v_cache, d.k_cache, d.v_cache), before


def _check_against_oracle(p, d, mix, before, prefill_rows=None, k_rel=0.0):
    """The mixed step's outputs and caches against the oracle: every decode request, and every prefill row (or
    the sampled `prefill_rows` per request)."""
    tol = tol_for(p.qkv.dtype)
    pk0, pv0, dk0, dv0 = before
    check_decode_result(d, mix[1], dk0, dv0, tol, "mixed-step decode", k_rel=k_rel)
    if prefill_rows is None:
        ref = oracle_prefill(p)
        assert_close(f64(mix[0]), ref["out"], tol, "mixed-step prefill out")
        check_prefill_caches(p, pk0, pv0, ref, tol, k_rel=k_rel)
        return
    qt, kt, v = oracle.qk_norm_rope(f64(p.qkv), f64(p.q_norm_weight), f64(p.k_norm_weight),
                                    p.positions.cpu().numpy(), **layer_kw(p.heads))
    check_prefill_caches(p, pk0, pv0, {"k_tilde": kt}, tol)
    cu = p.cu_seqlens.cpu().tolist()
    rows = sample_tokens(cu, prefill_rows, seed=15)
    want = oracle.prefill_rows(qt, kt, v, cu, rows)
    out = mix[0].reshape(p.num_tokens, p.heads.num_q_heads, p.heads.head_dim)
    got = f64(out.index_select(0, torch.tensor(rows, device=out.device)))
    err = assert_close(got, np.stack([want[n] for n in rows]), tol, f"mixed-step prefill, {len(rows)} sampled rows")
    note(f"mixed step: {len(rows)} sampled prefill rows x {p.heads.num_q_heads} heads, max-abs error {err:.3e}")
    assert len(rows) >= 512


def _assert_same(sep, mix):
    for name, a, b in zip(("prefill out", "decode out", "prefill K", "prefill V", "decode K", "decode V"), sep, mix):
        assert torch.equal(bits(a), bits(b)), f"{name} differs from the separate calls"
    assert torch.isfinite(mix[0].float()).all() and torch.isfinite(mix[1].float()).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (16, 16, 64), (16, 8, 128), (64, 8, 64), (16, 1, 128),
                                      (12, 4, 64)], ids=["g4d128", "g1d64", "g2d128", "g8d64", "g16d128", "g3d64"])
def test_mixed_step_equals_prefill_then_decode(hq, hkv, d, dtype):
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    lens = [300, 1, 0, 129]
    p = make_prefill_inputs(h, lens, seed=81, dtype=dtype, device=DEV, capacity=max(lens))
    dec = make_decode_inputs(h, [0, 5, 700, 3000, 31], seed=82, dtype=dtype, device=DEV)
    dec.q_norm_weight.copy_(p.q_norm_weight)
    dec.k_norm_weight.copy_(p.k_norm_weight)
    note(f"mixed step Hq {hq} Hkv {hkv} D {d} {dtype}")
    sep, mix, before = _both(p, dec)
    _assert_same(sep, mix)
    _check_against_oracle(p, dec, mix, before)


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (16, 16, 64), (64, 8, 64)], ids=["g4d128", "g1d64", "g8d64"])
def test_mixed_step_with_a_large_norm_weight(hq, hkv, d):
    """One weight element large enough that the scores are no longer bounded for the unshifted softmax: every
    prefill item of the fused launch returns at once and the running-max kernel that follows computes them."""
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    lens = [300, 1, 0, 129]
    p = make_prefill_inputs(h, lens, seed=85, device=DEV, capacity=max(lens))
    dec = make_decode_inputs(h, [0, 5, 700, 3000, 31], seed=86, device=DEV)
    wq, wk = f64(p.q_norm_weight), f64(p.k_norm_weight)
    wq[5], wk[d - 3] = 2.5, -2.5  # max|w_q| max|w_k| = 6.25, past the switch for D = 64 and 128
    p.q_norm_weight.copy_(torch.from_numpy(wq).to(p.q_norm_weight.dtype))
    p.k_norm_weight.copy_(torch.from_numpy(wk).to(p.k_norm_weight.dtype))
    dec.q_norm_weight.copy_(p.q_norm_weight)
    dec.k_norm_weight.copy_(p.k_norm_weight)
    note(f"mixed step Hq {hq} Hkv {hkv} D {d}, weights 2.5 / -2.5")
    sep, mix, before = _both(p, dec)
    _assert_same(sep, mix)
    _check_against_oracle(p, dec, mix, before, k_rel=2.0**-8)


def test_mixed_step_of_the_benchmark_workload():
    w = build_workload("mixed_qwen3_8b", device=DEV)
    note("mixed step: 4 x 4096 prefill + 128 decodes")
    sep, mix, before = _both(w.prefill, w.decode)
    _assert_same(sep, mix)
    # The fused launch's own results against the oracle: all 128 decode rows and their new slots, every prefill
    # cache entry, and sampled prefill rows of every head.
    _check_against_oracle(w.prefill, w.decode, mix, before, prefill_rows=136)


def test_mixed_step_with_an_empty_half():
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    for plens, dlens in (([0, 0], [40, 2]), ([70, 9], [])):
        p = make_prefill_inputs(h, plens, seed=83, device=DEV, capacity=max(plens + [1]))
        dec = make_decode_inputs(h, dlens or [0], seed=84, device=DEV)
        if not dlens:  # no decode requests at all
            dec.qkv, dec.positions, dec.cache_lens = dec.qkv[:0], dec.positions[:0], dec.cache_lens[:0]
            dec.k_cache, dec.v_cache = dec.k_cache[:0], dec.v_cache[:0]
        dec.q_norm_weight.copy_(p.q_norm_weight)
        dec.k_norm_weight.copy_(p.k_norm_weight)
        note(f"mixed step prefill {plens} decode {dlens}")
        sep, mix, _ = _both(p, dec)
        _assert_same(sep, mix)
