"""Host-side checks of bench.py's report (no GPU): the byte and roofline
arithmetic behind `value` and `roofline`, the automatic segment length the
long workload is timed with, when stored counter figures apply, and the
refusal of more than one GPU.

The expected byte counts are written out from the cost model (per
head-token q, k, v, g and out in bf16 plus the bf16 beta logit; per chain the
states; per head A_log and dt_bias), independently of bench.py's own
function.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import gated_delta_rule_36_amd as kda  # noqa: E402


def meta_inputs(B, T, H, *, init=None, cu_seqlens=None):
    """Shapes and dtypes of a workload without its data (meta tensors)."""
    bf = dict(dtype=torch.bfloat16, device="meta")
    q = torch.empty(B, T, H, 128, **bf)
    n = B if cu_seqlens is None else len(cu_seqlens) - 1
    return SimpleNamespace(
        q=q, k=q, v=q, g=q, beta=torch.empty(B, T, H, **bf),
        A_log=torch.empty(H, dtype=torch.float32, device="meta"),
        dt_bias=torch.empty(H, 128, dtype=torch.float32, device="meta"),
        initial_state=None if init is None else torch.empty(n, H, 128, 128, dtype=init, device="meta"),
        cu_seqlens=None if cu_seqlens is None else torch.tensor(cu_seqlens, dtype=torch.int64),
        num_seqs=n)


def expected_bytes(B, T, H, chains, init_bytes, final_bytes, n_cu=0):
    head_tokens = B * T * H
    per_head_token = 4 * 128 * 2 + 128 * 2 + 2  # q, k, v, g in; out; beta
    params = H * 4 + H * 128 * 4                 # A_log, dt_bias (fp32)
    states = chains * 128 * 128 * (init_bytes + final_bytes)
    return head_tokens * per_head_token + params + states + 8 * n_cu


def test_bytes_per_head_token_is_the_cost_model():
    assert 4 * 128 * 2 + 128 * 2 + 2 == 1282


@pytest.mark.parametrize("name,B,T,H,init,final,init_b,final_b", [
    ("tiny", 1, 64, 2, None, None, 0, 0),
    ("small", 2, 128, 8, None, None, 0, 0),
    ("long", 1, 8192, 16, torch.float32, torch.float32, 4, 4),
    ("large", 8, 16384, 32, None, torch.float32, 0, 4),
])
def test_algorithmic_bytes(name, B, T, H, init, final, init_b, final_b):
    x = meta_inputs(B, T, H, init=init)
    assert bench.algorithmic_bytes(x, final) == expected_bytes(B, T, H, B * H, init_b, final_b)


def test_algorithmic_bytes_of_the_large_workload():
    # the figure the roofline of the headline is quoted with
    assert bench.algorithmic_bytes(meta_inputs(8, 16384, 32), torch.float32) == 5_393_891_456


def test_algorithmic_bytes_packed_sequences():
    cu = [0, 100, 350, 1000]
    x = meta_inputs(1, 1000, 4, init=torch.bfloat16, cu_seqlens=cu)
    assert bench.algorithmic_bytes(x, torch.bfloat16) == expected_bytes(1, 1000, 4, 3 * 4, 2, 2, len(cu))


def test_roofline_fraction():
    x = meta_inputs(8, 16384, 32)
    r = bench.roofline_of(x, torch.float32, launch_ms=1.3481)
    achieved = 5_393_891_456 / 1.3481e-3 / 1e9
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(achieved, abs=0.05)
    assert r["frac"] == pytest.approx(achieved / 8000.0, abs=1e-4)
    assert r["frac"] == pytest.approx(0.5001, abs=1e-4)  # 50 % of 8 TB/s is 1.348 ms
    assert r["flops_per_launch"] == round(8 * 16384 * 32 * bench.FLOPS_PER_HEAD_TOKEN)


def test_segment_choice():
    def x(B, T, H):
        return SimpleNamespace(q=torch.empty(B, T, H, 128, device="meta"), num_seqs=B)
    assert bench.segment_choice(kda, x(1, 8192, 16), "auto") == 32   # 16 segments per chain
    assert bench.segment_choice(kda, x(8, 16384, 32), "auto") is None  # 256 chains fill the GPU
    assert bench.segment_choice(kda, x(1, 64, 2), "auto") is None      # too short to split
    assert bench.segment_choice(kda, x(1, 8192, 16), "off") is None
    assert bench.segment_choice(kda, x(1, 8192, 16), "12") == 12


def test_stored_traffic_applies_only_to_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"source_sha256": bench.source_digest(), "kernel_choice": "mfma",
           "hbm_bytes_per_launch": 123}
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("w", "mfma") == 123
    assert bench.stored_traffic("w", "single") is None
    assert bench.stored_traffic("absent", "mfma") is None
    (tmp_path / "traffic_w.json").write_text(json.dumps(dict(rec, source_sha256="0" * 64)))
    assert bench.stored_traffic("w", "mfma") is None


def test_committed_traffic_record_matches_the_sources():
    # the large workload's counters were taken on the kernel sources as committed
    with open(os.path.join(ROOT, "profiles", "traffic_large_b8_t16384_h32.json")) as fh:
        rec = json.load(fh)
    assert rec["source_sha256"] == bench.source_digest()
    assert rec["algorithmic_bytes_per_launch"] == 5_393_891_456
    assert 1.0 <= rec["traffic_over_algorithmic"] < 1.05


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "not supported" in r.stderr and r.stdout == ""


def test_launch_stats():
    st = bench.launch_stats([1.4, 1.38, 1.35, 1.33, 1.30, 1.29, 1.28, 1.27])
    assert st["first"] == 1.4 and st["min"] == 1.27 and st["max"] == 1.4
    assert st["median"] == 1.33  # the upper median of an even count
    assert st["first_quarter_mean"] == pytest.approx((1.4 + 1.38) / 2)
    assert st["last_quarter_mean"] == pytest.approx((1.28 + 1.27) / 2)
