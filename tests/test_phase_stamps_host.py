"""The phase-stamps profiling build on the host: its exports, and the summary arithmetic on a hand-made record."""

import ctypes
import pathlib
import re

import numpy as np

from decoder_attention_amd import phase_stamps
from decoder_attention_amd.build import LIB_PATH, STAMPS_LIB_PATH

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "qkra_phase_stamps.h"


def test_profiling_build_exports_every_declared_symbol():
    import decoder_attention_amd as da

    text = HEADER.read_text()
    names = sorted(set(re.findall(r"QKRA_STAMPS_API\s+[\w\s\*]*?\b(qkra_phase_stamps_\w+)\s*\(", text)))
    assert names == da.phase_stamps_symbols() and len(names) == 3
    lib = ctypes.CDLL(STAMPS_LIB_PATH)
    for name in names:
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value
    for name in da.exported_symbols():  # the attention ABI is the same library's
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value
    normal = ctypes.CDLL(LIB_PATH)
    assert not hasattr(normal, "qkra_phase_stamps_read")


def _record(items):
    """items: (cu, start, issued, q_ready, loop, first_step, loop_end, end, ntiles) in 100 MHz ticks."""
    rec = np.zeros((len(items) + 2, 8, 8), dtype=np.uint64)  # two workgroups that ran nothing stay zero
    for i, (cu, *ts, ntiles) in enumerate(items):
        for w in range(8):
            rec[i, w, :7] = ts
            rec[i, w, 7] = (cu << 8) | (ntiles << 20) | (i << 36)
    return rec


def test_summary_of_a_hand_made_record():
    # CU 1 runs two items back to back with a 2 us gap; CU 2 runs one and idles 50 us at the end.
    rec = _record([(1, 0, 300, 700, 900, 1100, 2100, 2200, 6),
                   (1, 2400, 2700, 3100, 3300, 3500, 4500, 4600, 6),
                   (2, 0, 300, 700, 900, 1100, 2100, 2200, 6)])
    res = phase_stamps.summarize(rec)
    assert res["workgroups"] == 3 and res["cus"] == 2 and res["workgroups_per_cu"] == 1.5
    assert abs(res["kernel_span_us"] - 46.0) < 1e-9
    it = res["per_item_us"]
    assert abs(it["issue_loads"]["mean"] - 3.0) < 1e-9 and abs(it["q_normalise_rotate"]["mean"] - 4.0) < 1e-9
    assert abs(it["prologue"]["mean"] - 9.0) < 1e-9 and abs(it["first_step"]["mean"] - 2.0) < 1e-9
    assert abs(it["later_step_each"]["mean"] - 2.0) < 1e-9  # 10 us over the 5 later steps
    assert abs(it["epilogue"]["mean"] - 1.0) < 1e-9
    cu = res["per_cu_us"]
    assert abs(cu["prologue"] - 13.5) < 1e-9      # (18 + 9) / 2
    assert abs(cu["gaps"] - 1.0) < 1e-9           # (2 + 0) / 2
    assert abs(cu["tail_idle"] - 12.0) < 1e-9     # (0 + 24) / 2
    md = phase_stamps.markdown("w", res, "cmd")
    assert "| prologue | 9.00 |" in md


def test_role_summary_of_a_fused_step_record():
    # Two decode-role workgroups (bit 63) on CUs 1 and 2, three prefill items on CUs 3, 3 and 1.
    rec = np.zeros((5, 8, 8), dtype=np.uint64)
    rows = [(0, 50000, True, 1), (0, 40000, True, 2), (100, 3000, False, 3), (3100, 9000, False, 3),
            (50100, 60000, False, 1)]
    for i, (st, en, dec, cu) in enumerate(rows):
        rec[i, :, 0] = st
        rec[i, :, 1:6] = [st + 10, st + 20, st + 30, st + 40, en - 10]
        rec[i, :, 6] = en
        rec[i, :, 7] = np.uint64((1 << 63) | (cu << 8)) if dec else np.uint64((cu << 8) | (3 << 20) | (i << 36))
    r = phase_stamps.summarize_roles(rec, bins=4)
    assert abs(r["span_us"] - 600.0) < 1e-9
    assert r["decode"]["workgroups"] == 2 and r["decode"]["cus"] == 2 and abs(r["decode"]["last_end_us"] - 500) < 1e-9
    assert r["prefill"]["workgroups"] == 3 and r["prefill"]["cus"] == 2
    assert abs(r["decode"]["busy_cu_us"] - 900.0) < 1e-9
    assert [round(x, 6) for x in r["cus_busy_by_slice"]["decode"]] == [2.0, 2.0, round(5 / 3, 6), round(1 / 3, 6)]
    assert phase_stamps.summarize(rec)["workgroups"] == 3  # the prefill items only
