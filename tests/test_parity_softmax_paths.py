"""Both softmax paths of the bf16 prefill, on the GPU against the oracle.

Softmax does not change when all scores of a row move by the same amount.
With RMS-normalised Q and K, every score is bounded by
max|w_q| * max|w_k| * sqrt(D) (Cauchy-Schwarz; the rotation keeps norms).
A request with no cached history whose norm weights keep that bound small
takes p = 2^s with no shift at all. Any other request subtracts a running row
max. The two paths are two kernels launched over the same grid. Each
workgroup decides from its request's history length and the weights which of
them computes its rows.

- Largest weights just below and just above the switch give oracle results, and
  every output row is written: `out` starts as NaN, so a row that neither
  kernel, or the wrong one, handled would show.
- Q heads equal to their K head, with weights 4, put each row's own score near
  2^261. Unshifted, p would overflow to inf and the row would be NaN, so this
  case passes only when the shifted kernel ran.
"""

import numpy as np
import pytest
import torch

import decoder_attention_amd as da
from harness import BF16_TOL, assert_close, cfg_of, f64, note, oracle_prefill
from workloads import HeadConfig, make_prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _set_weights(p, wq: np.ndarray, wk: np.ndarray) -> None:
    p.q_norm_weight.copy_(torch.from_numpy(wq).to(p.q_norm_weight.dtype))
    p.k_norm_weight.copy_(torch.from_numpy(wk).to(p.k_norm_weight.dtype))


def _run_and_check(p, what: str) -> None:
    h = p.heads
    out = torch.full((p.num_tokens, h.num_q_heads * h.head_dim), float("nan"), dtype=p.qkv.dtype, device=DEV)
    da.prefill(cfg_of(h, p.qkv.dtype), p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens,
               p.max_seqlen, p.k_cache, p.v_cache, out=out)
    torch.cuda.synchronize()
    ref = oracle_prefill(p)
    assert_close(f64(out), ref["out"], BF16_TOL, f"{what}: out")
    # K cache: the bound 2e-2 plus half a bf16 step of the value (k~ reaches
    # |x| >= 8 here, where one correctly rounded bf16 is off by up to 0.03).
    cu = p.cu_seqlens.cpu().tolist()
    for r in range(p.num_seqs):
        lo, hi = cu[r], cu[r + 1]
        got = f64(p.k_cache[r, :, : hi - lo])
        want = np.transpose(ref["k_tilde"][lo:hi], (1, 0, 2))
        assert np.all(np.abs(got - want) <= BF16_TOL + np.abs(want) * 2.0**-8), f"{what}: K cache request {r}"


# One element of each weight vector set to c (the rest drawn as usual, |w| < 1.5), so that
# max|w_q| max|w_k| = c^2.  The switch lies at 48 / (1.02 D log2(e) / sqrt(D)): 2.88 for D = 128
# (c = 1.697) and 4.08 for D = 64 (c = 2.019); each list has bf16 values on both sides.  Uniform
# weights that large would amplify every score about 2.9x, and the bf16 rounding of q~ and k~ alone
# would then exceed the bound on either path.
@pytest.mark.parametrize("head_dim,hq,hkv,weights", [
    (128, 32, 8, [1.6875, 1.6953125, 1.703125, 1.7109375]),
    (64, 8, 2, [2.0, 2.015625, 2.03125, 2.046875]),
    (128, 16, 16, [1.6953125, 1.703125]),
], ids=["d128_g4", "d64_g4", "d128_g1"])
def test_weights_on_both_sides_of_the_switch(head_dim, hq, hkv, weights):
    h = HeadConfig(hq, hkv, head_dim, 1e-6, 1e6)
    lens = [300, 1, 0, 129]
    for c in weights:
        p = make_prefill_inputs(h, lens, seed=61, device=DEV, capacity=max(lens))
        wq, wk = f64(p.q_norm_weight), f64(p.k_norm_weight)
        assert np.abs(wq).max() < c and np.abs(wk).max() < c
        wq[3], wk[3] = c, -c
        _set_weights(p, wq, wk)
        note(f"prefill D={head_dim} Hq={hq} Hkv={hkv} largest weights {c}")
        _run_and_check(p, f"weights {c}")


def test_one_large_weight_takes_the_shifted_path():
    """The bound uses the largest weight: one outlier element moves the switch, while the typical scores stay
    moderate."""
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    lens = [513, 64, 7]
    p = make_prefill_inputs(h, lens, seed=62, device=DEV, capacity=max(lens))
    wq, wk = f64(p.q_norm_weight), f64(p.k_norm_weight)
    wq[5], wk[77] = 2.5, -2.5
    _set_weights(p, wq, wk)
    note("prefill with one outlier weight per norm")
    _run_and_check(p, "outlier weights")


@pytest.mark.parametrize("head_dim", [128, 64])
def test_scores_beyond_fp32_range_need_the_shift(head_dim):
    h = HeadConfig(8, 2, head_dim, 1e-6, 1e4)
    lens = [200, 75]
    p = make_prefill_inputs(h, lens, seed=63, device=DEV, capacity=max(lens))
    g = h.num_q_heads // h.num_kv_heads
    d = head_dim
    for q in range(h.num_q_heads):  # Q head q := its K head, so q~ = k~ at every token
        kv = h.num_q_heads + q // g
        p.qkv[:, q * d:(q + 1) * d] = p.qkv[:, kv * d:(kv + 1) * d]
    _set_weights(p, np.full(d, 4.0), np.full(d, 4.0))
    note(f"prefill D={head_dim} with q = k and weights 4 (self scores ~2^261)")
    _run_and_check(p, "q = k, weights 4")


# ---- the caller's weight bound (qkra_config.qk_weight_bound) -------------------------------------------------
# With a bound the host launches only the softmax kernel the bound selects.  Launches are counted with the
# library's kernel timing (ids 1: unshifted, 10: running max).

def _launches(fn):
    da.qknorm_rope_attn_set_kernel_timing((1 << 1) | (1 << 10))
    da.qknorm_rope_attn_read_kernel_timing()
    fn()
    torch.cuda.synchronize()
    k = da.qknorm_rope_attn_read_kernel_timing()
    da.qknorm_rope_attn_set_kernel_timing(False)
    return {name: n for name, (_, n) in k.items()}


def _prefill_out(p, bound):
    h = p.heads
    cfg = da.make_config(h.num_q_heads, h.num_kv_heads, h.head_dim, p.qkv.dtype, h.rms_eps, h.rope_base,
                         qk_weight_bound=bound)
    out = torch.full((p.num_tokens, h.num_q_heads * h.head_dim), float("nan"), dtype=p.qkv.dtype, device=DEV)
    launches = _launches(lambda: da.prefill(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions,
                                            p.cu_seqlens, p.max_seqlen, p.k_cache, p.v_cache, out=out))
    return out, launches


@pytest.mark.parametrize("head_dim", [128, 64])
def test_weight_bound_launches_one_kernel(head_dim):
    h = HeadConfig(16, 4, head_dim, 1e-6, 1e6)
    lens = [300, 1, 0, 129]
    p = make_prefill_inputs(h, lens, seed=64, device=DEV, capacity=max(lens))
    wq, wk = f64(p.q_norm_weight), f64(p.k_norm_weight)
    prod = float(np.abs(wq).max() * np.abs(wk).max())
    limit = da.qknorm_rope_attn_unshifted_weight_limit(head_dim)
    assert prod < limit
    base, both = _prefill_out(p, 0.0)                       # no bound: both kernels launched
    assert both == {"prefill_attn_mfma_bf16": 1, "prefill_attn_mfma_bf16_shifted": 1}
    small, one = _prefill_out(p, prod * 1.01)               # a true bound under the limit: the unshifted kernel
    assert one == {"prefill_attn_mfma_bf16": 1}
    assert torch.equal(small.view(torch.int16), base.view(torch.int16))
    large, one = _prefill_out(p, limit * 2)                 # a bound past the limit: the running-max kernel only
    assert one == {"prefill_attn_mfma_bf16_shifted": 1}
    ref = oracle_prefill(p)
    assert_close(f64(large), ref["out"], BF16_TOL, "running-max kernel for every item")
    note(f"D={head_dim}: weight bound {prod:.3f} (limit {limit:.3f}): one launch, same bits")


def test_weight_bound_broken_by_the_weights_gives_nan_rows():
    """A bound that selects the unshifted softmax while the weights exceed the limit: no kernel can compute the
    rows, and they are written as NaN rather than left as whatever the buffer held."""
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    lens = [70, 5]
    p = make_prefill_inputs(h, lens, seed=65, device=DEV, capacity=max(lens))
    wq, wk = f64(p.q_norm_weight), f64(p.k_norm_weight)
    wq[5], wk[77] = 2.5, -2.5
    _set_weights(p, wq, wk)
    h2 = p.heads
    cfg = da.make_config(h2.num_q_heads, h2.num_kv_heads, h2.head_dim, p.qkv.dtype, h2.rms_eps, h2.rope_base,
                         qk_weight_bound=1.0)
    out = torch.zeros((p.num_tokens, 32 * 128), dtype=p.qkv.dtype, device=DEV)
    launches = _launches(lambda: da.prefill(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions,
                                            p.cu_seqlens, p.max_seqlen, p.k_cache, p.v_cache, out=out))
    assert launches == {"prefill_attn_mfma_bf16": 1}
    assert torch.isnan(out.float()).all(), "rows the broken bound left uncomputed must be NaN"


def test_weight_bound_in_the_mixed_step():
    """The mixed step with a true bound: no running-max launch after the fused one, and the same bits."""
    from workloads import make_decode_inputs

    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    p = make_prefill_inputs(h, [300, 1, 129], seed=66, device=DEV, capacity=300)
    d = make_decode_inputs(h, [5, 700, 3000], seed=67, device=DEV)
    d.q_norm_weight.copy_(p.q_norm_weight)
    d.k_norm_weight.copy_(p.k_norm_weight)
    prod = float(np.abs(f64(p.q_norm_weight)).max() * np.abs(f64(p.k_norm_weight)).max())
    outs = []
    for bound, want in ((0.0, {"prefill_attn_mfma_bf16_shifted": 1}), (prod, {})):
        cfg = da.make_config(32, 8, 128, torch.bfloat16, 1e-6, 1e6, qk_weight_bound=bound)
        pk, pv, dk, dv = p.k_cache.clone(), p.v_cache.clone(), d.k_cache.clone(), d.v_cache.clone()
        res = {}

        def run():
            res["out"] = da.mixed_step(cfg, p.q_norm_weight, p.k_norm_weight, p.qkv, p.positions, p.cu_seqlens,
                                       p.max_seqlen, pk, pv, d.qkv, d.positions, d.cache_lens, d.max_cache_len, dk,
                                       dv)
        assert _launches(run) == want
        outs.append(res["out"][:2])
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


# ---- the finite V range each path guarantees (include/qknorm_rope_attn.h) ---------------------------------
# Softmax weights do not depend on V, so every output is linear in V: scaling V by 2^e scales each product,
# partial sum, row total and the bf16 rounding of the output by exactly 2^e while nothing overflows.  At the
# stated limits (keys per row times max|V| below 2^79 without a shift, below 2^119 with the running max) the
# rows stay finite and equal the unscaled ones times 2^e, bit for bit.

def _scaled_v(qkv, h, e):
    out = qkv.clone()
    v0 = (h.num_q_heads + h.num_kv_heads) * h.head_dim
    out[:, v0:] = (out[:, v0:].float() * 2.0**e).to(out.dtype)
    return out


@pytest.mark.parametrize("path,e", [("unshifted", 64), ("running_max", 104)])
def test_prefill_v_range_scales_exactly(path, e):
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    lens = [2048, 300]  # up to 2^11 keys per row; drawn |v| < 2^3
    p = make_prefill_inputs(h, lens, seed=68, device=DEV, capacity=max(lens))
    prod = float(np.abs(f64(p.q_norm_weight)).max() * np.abs(f64(p.k_norm_weight)).max())
    bound = prod if path == "unshifted" else 2 * da.qknorm_rope_attn_unshifted_weight_limit(128)
    assert float(p.qkv.float().abs().max()) < 8 and (2048 * 8 * 2.0**e < 2.0**(79 if path == "unshifted" else 119))
    cfg = da.make_config(32, 8, 128, torch.bfloat16, 1e-6, 1e6, qk_weight_bound=bound)
    outs, vcs = [], []
    for scale in (0, e):
        qkv = _scaled_v(p.qkv, h, scale)
        kc, vc = p.k_cache.clone(), p.v_cache.clone()
        launches = _launches(lambda: outs.append(da.prefill(cfg, qkv, p.q_norm_weight, p.k_norm_weight, p.positions,
                                                            p.cu_seqlens, p.max_seqlen, kc, vc)[0]))
        assert launches == {"prefill_attn_mfma_bf16" + ("" if path == "unshifted" else "_shifted"): 1}
        vcs.append(vc)
    base, scaled = outs
    assert torch.isfinite(scaled.float()).all()
    want = (base.float() * 2.0**e).to(torch.bfloat16)
    assert torch.equal(scaled.view(torch.int16), want.view(torch.int16)), f"{path}: out scales by 2^{e} exactly"
    for r, L in enumerate(lens):
        got = vcs[1][r, :, :L].float()
        assert torch.equal(got, vcs[0][r, :, :L].float() * 2.0**e)
    note(f"prefill {path}: V x 2^{e} gives out x 2^{e} bit for bit")


def test_decode_v_range_scales_exactly():
    from workloads import make_decode_inputs

    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    e = 104  # 3001 keys * |v| < 8 * 2^104 < 2^119
    d = make_decode_inputs(h, [5, 700, 3000], seed=69, device=DEV)
    cfg = da.make_config(32, 8, 128, torch.bfloat16, 1e-6, 1e6)
    outs = []
    for scale in (0, e):
        qkv = _scaled_v(d.qkv, h, scale)
        kc, vc = d.k_cache.clone(), d.v_cache.clone()
        for b, L in enumerate([5, 700, 3000]):
            vc[b, :, :L] = (vc[b, :, :L].float() * 2.0**scale).to(vc.dtype)
        outs.append(da.decode(cfg, qkv, d.q_norm_weight, d.k_norm_weight, d.positions, d.cache_lens,
                              d.max_cache_len, kc, vc)[0])
    torch.cuda.synchronize()
    assert torch.isfinite(outs[1].float()).all()
    want = (outs[0].float() * 2.0**e).to(torch.bfloat16)
    assert torch.equal(outs[1].view(torch.int16), want.view(torch.int16)), "decode: out scales by 2^104 exactly"
    assert float(d.qkv.float().abs().max()) < 8
    assert all(float(d.v_cache[b, :, :L].float().abs().max()) < 8 for b, L in enumerate([5, 700, 3000]))
    note("decode: V x 2^104 gives out x 2^104 bit for bit")
