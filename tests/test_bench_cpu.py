"""Host logic of bench.py: the algorithmic byte and flop counts of the
roofline, and which counter record may be attached to a bench line."""
import json

import pytest

import bench


def test_prefill_bytes_per_token_head():
    # q, k (bf16, d_k), v (bf16, d_v), g (fp32, d_k), beta (fp32), o (bf16,
    # d_v): 768 + 512 + 4 + 256 = 1540 B per token-head at d = 128
    assert bench.prefill_bytes(1, 1, 128, 128, 0, False) == 1540
    # S_T written per (sequence, head); S0 read as well when given
    st = 128 * 128 * 4
    assert bench.prefill_bytes(0, 2, 128, 128, 3, False) == 6 * st
    assert bench.prefill_bytes(0, 2, 128, 128, 3, True) == 12 * st
    # the bench workload: 4 x 4096 tokens, H = 32, S0 = 0
    assert bench.prefill_bytes(16384, 32, 128, 128, 4, False) == 815792128


def test_prefill_flops_per_token_head():
    assert bench.prefill_flops(1, 1, 128, 128) == 6 * 128 * 128 + 16 * (3 * 128 + 2 * 128)
    assert bench.prefill_flops(1, 1, 128, 128) == 108544


def test_decode_bytes():
    state, total = bench.decode_bytes(256, 64, 128, 128)
    assert state == 256 * 64 * 128 * 128 * 4 * 2
    assert total - state == 256 * 64 * 1540


@pytest.fixture
def record(tmp_path, monkeypatch):
    path = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PROFILE_PMC", str(path))

    def write(**kw):
        rec = {"kernel": "kda_prefill_kernel", "workload": "prefill",
               "hbm_bytes_per_launch": 123.0,
               "kernel_source_sha256_16": bench.source_hash()}
        rec.update(kw)
        path.write_text(json.dumps(rec))
    return write


def test_traffic_only_for_matching_source_and_workload(record):
    record()
    assert bench.measured_traffic("prefill") == 123.0
    # counters taken on the prefill workload say nothing about other workloads
    assert bench.measured_traffic("long_prefill") is None
    assert bench.measured_traffic("varlen") is None
    # a record taken on other kernel sources is stale
    record(kernel_source_sha256_16="0" * 16)
    assert bench.measured_traffic("prefill") is None
    # a record that does not name its workload is not trusted
    record(workload=None)
    assert bench.measured_traffic("prefill") is None


def test_traffic_missing_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_PMC", str(tmp_path / "absent.json"))
    assert bench.measured_traffic("prefill") is None

