"""qknorm_rope_attn_mixed_step on the GPU: a prefill batch and a decode batch in one call.

It computes what qknorm_rope_attn_prefill followed by qknorm_rope_attn_decode computes. In bf16, for the
head groupings it supports, it runs the prefill attention and the decode split in one launch. The decode role
runs the same wavefronts over the same plan as the decode split, and the prefill role the same work items, so
every output and cache must equal the two separate calls bit for bit. Outputs start as NaN, so a row that no
workgroup wrote shows. Groupings outside the supported set (G = 3 here) and fp32 take the two calls in turn.
"""

import pytest
import torch

import decoder_attention_amd as da
from harness import assert_close, bits, cfg_of, f64, note, oracle_prefill
from workloads import HeadConfig, build_workload, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _both(p, d):
    """Separate calls on clones of the caches, then the mixed step on the originals; returns both results."""
    h = p.heads
    cfg = cfg_of(h, p.qkv.dtype)
    width = h.num_q_heads * h.head_dim
    pk, pv, dk, dv = p.k_cache.clone(), p.v_cache.clone(), d.k_cache.clone(), d.v_cache.clone()
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
    return (sep_p, sep_d, pk, pv, dk, dv), (mix_p, mix_d, p.k_cache, p.v_cache, d.k_cache, d.v_cache)


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
    sep, mix = _both(p, dec)
    _assert_same(sep, mix)
    if hq == 32 and dtype == torch.bfloat16:  # and against the oracle once
        ref = oracle_prefill(p)
        assert_close(f64(mix[0]), ref["out"], 2e-2, "prefill out")


def test_mixed_step_of_the_benchmark_workload():
    w = build_workload("mixed_qwen3_8b", device=DEV)
    note("mixed step: 4 x 4096 prefill + 128 decodes")
    sep, mix = _both(w.prefill, w.decode)
    _assert_same(sep, mix)


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
        sep, mix = _both(p, dec)
        _assert_same(sep, mix)
