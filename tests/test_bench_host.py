"""bench.py's host-side logic, on the CPU: the work it divides by, which prefill kernel it reports, the
traffic lookup, and the refusal of more than one GPU."""

import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_prefill_flops_count_the_causal_pairs():
    # 4*D FLOP per allowed (query, key) pair and head; request of T tokens has T(T+1)/2 pairs.
    assert bench.prefill_flops([3], hq=2, d=8) == 4 * 8 * 2 * (3 * 4 // 2)
    # The 32k single-request prefill with 32 query heads of 128: 8.796e12 FLOP.
    assert bench.prefill_flops([32768], 32, 128) == pytest.approx(8.796e12, rel=1e-4)
    assert bench.prefill_flops([0, 5], 4, 64) == bench.prefill_flops([5], 4, 64)


def test_append_flops_reduce_to_prefill_without_history():
    assert bench.append_flops([0, 0], [7, 300], 32, 128) == bench.prefill_flops([7, 300], 32, 128)
    # One token onto P cached entries sees P + 1 keys.
    assert bench.append_flops([10], [1], 4, 64) == 4 * 64 * 4 * 11


def test_decode_bytes_read_each_kv_head_once():
    # K and V of every KV head, L_b + 1 entries each (the new token included), 2 bytes per bf16.
    assert bench.decode_kv_bytes([0, 9], hkv=8, d=128, elem=2) == 2 * 8 * 128 * 2 * (1 + 10)


def test_working_prefill_kernel_is_the_one_that_ran():
    k = {"prefill_attn_mfma_bf16": (5.0, 10), "prefill_attn_mfma_bf16_shifted": (0.1, 10)}
    assert bench.working_prefill_kernel(k) == "prefill_attn_mfma_bf16"
    k = {"prefill_attn_mfma_bf16": (0.1, 10), "prefill_attn_mfma_bf16_shifted": (24.0, 10)}
    assert bench.working_prefill_kernel(k) == "prefill_attn_mfma_bf16_shifted"
    assert bench.working_prefill_kernel({"decode_attn_split": (1.0, 1)}) is None


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    src = ["decoder_attention_amd/csrc/decode_mfma.hip"]
    table = {"decode_attn_split": {
        "w_now": {"hbm_bytes_per_launch": 123.0, "source_sha256": bench.source_digest(src)},
        "w_old": {"hbm_bytes_per_launch": 456.0, "source_sha256": "0" * 64}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(table))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "decode_attn_split", src)
    assert bench.measured_traffic("decode_attn_split", "w_now") == 123.0
    assert bench.measured_traffic("decode_attn_split", "w_old") is None
    assert bench.measured_traffic("decode_attn_split", "absent") is None
    assert bench.measured_traffic("unknown_kernel", "w_now") is None


def test_every_timed_kernel_names_existing_sources():
    for name, paths in bench.KERNEL_SOURCES.items():
        for p in paths:
            assert os.path.exists(os.path.join(ROOT, p)), (name, p)


def test_more_than_one_gpu_is_refused_before_any_gpu_work(capsys, monkeypatch):
    monkeypatch.delenv("WORLD_SIZE", raising=False)
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
    monkeypatch.setenv("WORLD_SIZE", "4")
    assert bench.main([]) == 2
