"""The steps next to the attention layer, on the GPU through the C ABI, against the fp64 oracle:
fused residual add + RMSNorm, last-position gather, greedy argmax."""

import numpy as np
import pytest
import torch

import decoder_attention_amd as da
import oracle
from harness import BF16_TOL, FP32_TOL, bits, f64, note
from workloads import build_workload, make_next_token_inputs, make_norm_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def norm_tol(ref: np.ndarray, dtype) -> np.ndarray:
    # bf16: the stated 2e-2 bound, widened to one bf16 ulp of the reference
    # (rounding a value of magnitude m to bf16 alone costs up to m * 2^-9).
    if dtype == torch.float32:
        return np.full(ref.shape, FP32_TOL)
    return np.maximum(BF16_TOL, np.abs(ref) * 2.0 ** -8)


def check_norm(n, dtype, out, res_after, x0, res0, eps, rows=None):
    rows = np.arange(out.shape[0]) if rows is None else np.asarray(rows)
    want_out, want_res = oracle.fused_add_rms_norm(f64(x0[rows]), None if res0 is None else f64(res0[rows]),
                                                   f64(n.weight), eps)
    got = f64(out[rows])
    err = np.abs(got - want_out)
    assert (err <= norm_tol(want_out, dtype)).all(), f"out: max-abs error {err.max():.3e}"
    # The new residual: the sum rounded to fp32, then stored in the dtype.
    stored = want_res.astype(np.float32).astype(np.float64)
    if dtype == torch.bfloat16:
        stored = oracle.round_to_bf16(stored)
    assert np.array_equal(f64(res_after[rows]), stored), "residual bits differ from the rounded sum"
    return float(err.max())


NORM_CASES = [(1, 8), (3, 1024), (67, 2560), (5, 4096), (2, 5120), (33, 2056), (4, 32768)]


@pytest.mark.parametrize("has_residual", [True, False], ids=["add", "first"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("rows,hidden", NORM_CASES, ids=[f"n{r}-c{c}" for r, c in NORM_CASES])
def test_fused_add_rmsnorm_matches_oracle(rows, hidden, dtype, has_residual):
    note(f"fused_add_rmsnorm rows={rows} hidden={hidden} {dtype} residual={has_residual}")
    n = make_norm_inputs(rows, hidden, seed=rows * 131 + hidden, dtype=dtype, device=DEV, has_residual=has_residual)
    x0 = n.x.clone()
    res0 = n.residual.clone() if has_residual else None
    res = n.residual if has_residual else torch.full_like(n.x, float("nan"))
    out = da.fused_add_rmsnorm(n.x, res, n.weight, n.rms_eps, has_residual)
    torch.cuda.synchronize()
    assert torch.equal(bits(n.x), bits(x0)), "x changed"
    check_norm(n, dtype, out, res, x0, res0, n.rms_eps)


def test_fused_add_rmsnorm_in_place_and_shared_residual():
    # out == x (in place), and a first call whose residual buffer is x itself.
    n = make_norm_inputs(9, 4096, seed=5, device=DEV)
    x0, res0 = n.x.clone(), n.residual.clone()
    out = da.fused_add_rmsnorm(n.x, n.residual, n.weight, n.rms_eps, True, out=n.x)
    torch.cuda.synchronize()
    assert out.data_ptr() == n.x.data_ptr()
    check_norm(n, torch.bfloat16, out, n.residual, x0, res0, n.rms_eps)
    m = make_norm_inputs(9, 4096, seed=6, device=DEV, has_residual=False)
    x1 = m.x.clone()
    out = da.fused_add_rmsnorm(m.x, m.x, m.weight, m.rms_eps, False)
    torch.cuda.synchronize()
    assert torch.equal(bits(m.x), bits(x1))
    check_norm(m, torch.bfloat16, out, m.x, x1, None, m.rms_eps)


def test_fused_add_rmsnorm_two_layer_chain():
    # The pages' layer loop with the fused call: first norm, sublayer stand-in,
    # second norm adding it to the residual; against the oracle's same chain.
    n = make_norm_inputs(40, 1024, seed=7, device=DEV, has_residual=False)
    res = torch.empty_like(n.x)
    y1 = da.fused_add_rmsnorm(n.x, res, n.weight, n.rms_eps, False)
    torch.cuda.synchronize()
    sub = (y1.float() * 0.5).to(torch.bfloat16)  # stand-in sublayer output
    y2 = da.fused_add_rmsnorm(sub, res, n.weight, n.rms_eps, True)
    torch.cuda.synchronize()
    o1, r1 = oracle.fused_add_rms_norm(f64(n.x), None, f64(n.weight), n.rms_eps)
    o2, r2 = oracle.fused_add_rms_norm(f64(sub), r1, f64(n.weight), n.rms_eps)
    err = np.abs(f64(y2) - o2)
    assert (err <= norm_tol(o2, torch.bfloat16)).all(), f"max-abs error {err.max():.3e}"


def test_fused_add_rmsnorm_mixed_step_sampled():
    # The benchmark's shape: 16512 rows of 4096.  Every row's residual is checked
    # bit for bit; the normalised output on sampled rows (first, last, random).
    w = build_workload("residual_rmsnorm_qwen3_8b", device=DEV)
    n = w.norm
    x0, res0 = n.x.clone(), n.residual.clone()
    out = da.fused_add_rmsnorm(n.x, n.residual, n.weight, n.rms_eps, True)
    torch.cuda.synchronize()
    stored = oracle.round_to_bf16((f64(x0) + f64(res0)).astype(np.float32).astype(np.float64))
    assert np.array_equal(f64(n.residual), stored)
    rng = np.random.default_rng(8)
    rows = sorted({0, n.x.shape[0] - 1} | set(rng.choice(n.x.shape[0], 62, replace=False).tolist()))
    err = check_norm(n, torch.bfloat16, out, n.residual, x0, res0, n.rms_eps, rows)
    note(f"fused add + RMSNorm, 16512x4096: sampled rows max-abs error {err:.3e}")


# ---- last-position gather -----------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gather_last_matches_oracle(dtype):
    seqlens = [3, 0, 1, 7, 0, 2]
    nt = make_next_token_inputs(seqlens, 264, 16, seed=9, dtype=dtype, device=DEV)
    out = torch.full((len(seqlens), 264), 4096.0, dtype=dtype, device=DEV)  # exact in bf16 and fp32
    da.gather_last(nt.hidden, nt.cu_seqlens, out=out)
    torch.cuda.synchronize()
    want = oracle.gather_last(f64(nt.hidden), nt.cu_seqlens.cpu().numpy())
    got = f64(out)
    for r, t in enumerate(seqlens):
        if t == 0:
            assert (got[r] == 4096.0).all(), f"row of empty request {r} was written"
        else:
            assert np.array_equal(got[r], want[r]), f"request {r}"


def test_gather_last_mixed_step():
    nt = build_workload("next_token_qwen3_8b", device=DEV).next_token
    out = da.gather_last(nt.hidden, nt.cu_seqlens)
    torch.cuda.synchronize()
    want = oracle.gather_last(f64(nt.hidden), nt.cu_seqlens.cpu().numpy())
    assert np.array_equal(f64(out), want)


# ---- greedy argmax ------------------------------------------------------------

def run_argmax(logits):
    out = da.argmax(logits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64)


ARGMAX_CASES = [(1, 1), (1, 7), (3, 8), (5, 100), (4, 2049), (7, 32000), (2, 151936), (3, 151937)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("rows,vocab", ARGMAX_CASES, ids=[f"b{b}-v{v}" for b, v in ARGMAX_CASES])
def test_argmax_matches_oracle(rows, vocab, dtype):
    note(f"argmax rows={rows} vocab={vocab} {dtype}")
    g = torch.Generator().manual_seed(rows * 7 + vocab)
    stride = (vocab + 7) // 8 * 8 + (8 if vocab % 3 == 0 else 0)  # padded rows for some cases
    buf = torch.randn((rows, stride), generator=g).to(dtype).to(DEV)
    logits = buf[:, :vocab]
    want = oracle.greedy_argmax(f64(logits))
    assert np.array_equal(run_argmax(logits), want)


def test_argmax_ties_nan_and_infinities():
    v = 151936
    z = torch.full((6, v), -1.0)
    z[0, [5000, 100000, 151935]] = 10.0                    # ties across segments: lowest index
    z[1, 7], z[1, 140000] = float("nan"), float("inf")     # NaN beats +inf
    z[2, [90000, 12]] = float("nan")                       # first NaN
    z[3] = -float("inf")                                   # all -inf: index 0
    z[4, v - 1] = 3.0                                      # maximum in the last element
    z[5, 20000:20008] = 2.0                                # a run of equal maxima
    for dtype in (torch.bfloat16, torch.float32):
        got = run_argmax(z.to(dtype).to(DEV))
        assert list(got) == [5000, 7, 12, 0, v - 1, 20000], (dtype, list(got))
        assert np.array_equal(got, oracle.greedy_argmax(f64(z.to(dtype))))


def test_argmax_mixed_step_sampled():
    # The benchmark's shape: 132 rows of 151936 bf16 logits.  The oracle's scan on
    # sampled rows; every row against the library argmax (first occurrence).
    nt = build_workload("next_token_qwen3_8b", device=DEV).next_token
    got = run_argmax(nt.logits)
    rows = [0, 3, 4, 77, 131]
    want = oracle.greedy_argmax(f64(nt.logits[rows]))
    assert np.array_equal(got[rows], want)
    assert np.array_equal(got, np.argmax(f64(nt.logits), axis=1))


# ---- seeded sweep ---------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("i", range(8))
def test_fused_add_rmsnorm_sweep(i, dtype):
    # Random row counts and hidden sizes (any multiple of 8 up to 32768), eps, first or later call.
    rng = np.random.default_rng(500 + i)
    rows = int(rng.integers(1, 300))
    hidden = 8 * int(rng.integers(1, 4097))
    has_residual = bool(rng.integers(0, 2))
    eps = float(rng.choice([1e-6, 1e-5, 1e-2]))
    note(f"fused_add_rmsnorm sweep {i}: rows {rows} hidden {hidden} residual {has_residual} eps {eps} {dtype}")
    n = make_norm_inputs(rows, hidden, seed=int(rng.integers(1 << 20)), dtype=dtype, device=DEV,
                         has_residual=has_residual, rms_eps=eps)
    x0 = n.x.clone()
    res0 = n.residual.clone() if has_residual else None
    res = n.residual if has_residual else torch.empty_like(n.x)
    out = da.fused_add_rmsnorm(n.x, res, n.weight, eps, has_residual)
    torch.cuda.synchronize()
    check_norm(n, dtype, out, res, x0, res0, eps)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("i", range(8))
def test_argmax_sweep(i, dtype):
    # Random vocabularies (not multiples of anything), padded strides, planted ties and extremes.
    rng = np.random.default_rng(600 + i)
    rows = int(rng.integers(1, 12))  # the oracle scans in Python
    vocab = int(rng.integers(1, 200000))
    stride = (vocab + 7) // 8 * 8 + 8 * int(rng.integers(0, 3))
    g = torch.Generator().manual_seed(int(rng.integers(1 << 20)))
    buf = torch.randn((rows, stride), generator=g)
    for r in range(rows):  # a planted maximum, sometimes repeated (ties go to the lowest index)
        at = rng.integers(0, vocab, size=int(rng.integers(1, 4)))
        buf[r, at] = 50.0
    logits = buf.to(dtype).to(DEV)[:, :vocab]
    note(f"argmax sweep {i}: rows {rows} vocab {vocab} stride {stride} {dtype}")
    want = oracle.greedy_argmax(f64(logits))
    assert np.array_equal(run_argmax(logits), want)
